// Select kernels for key tile 128 (4 waves x 1 blocks x 1 register tiles), bf16 keys.
#include "si_select.hpp"

namespace si {
template hipError_t launch_select_shape<4, 1, 1, false>(const SelectArgs&, int,
                                                              hipStream_t);
}  // namespace si
