// Dispatch of the select stage to the kernel of the planned register-tile shape.
#include "si_kernels.hpp"

namespace si {

hipError_t launch_select(const SelectArgs& a, int nwave, int kb, int nsub, int cg, int op,
                         hipStream_t stream) {
#define SI_SHAPE(NW, KB, NS)                                                          \
    if (nwave == NW && kb == KB && nsub == NS) {                                      \
        switch (op) {                                                                 \
            case kOpBf16: return launch_select_shape<NW, KB, NS, kOpBf16>(a, cg, stream);     \
            case kOpBf16K8: return launch_select_shape<NW, KB, NS, kOpBf16K8>(a, cg, stream); \
            case kOpF8: return launch_select_shape<NW, KB, NS, kOpF8>(a, cg, stream);         \
            case kOpF8K4: return launch_select_shape<NW, KB, NS, kOpF8K4>(a, cg, stream);     \
            default: return hipErrorInvalidValue;                                     \
        }                                                                             \
    }
    SI_SHAPE(2, 1, 1)
    SI_SHAPE(4, 1, 1)
    SI_SHAPE(4, 2, 1)
    SI_SHAPE(4, 4, 1)
    SI_SHAPE(4, 2, 3)
    SI_SHAPE(4, 4, 2)
#undef SI_SHAPE
    return hipErrorInvalidValue;
}

}  // namespace si
