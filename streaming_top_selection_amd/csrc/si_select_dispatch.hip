// Dispatch of the select stage to the kernel of the planned register-tile shape.
#include "si_kernels.hpp"

namespace si {

hipError_t launch_select(const SelectArgs& a, int nwave, int kb, int nsub, int cg, bool fp8,
                         hipStream_t stream) {
#define SI_SHAPE(NW, KB, NS)                                                          \
    if (nwave == NW && kb == KB && nsub == NS)                                        \
        return fp8 ? launch_select_shape<NW, KB, NS, true>(a, cg, stream)             \
                   : launch_select_shape<NW, KB, NS, false>(a, cg, stream);
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
