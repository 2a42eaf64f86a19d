// Select kernels for key tile 1024 (4 waves x 4 blocks x 2 register tiles), bf16 keys.
#include "si_select.hpp"

namespace si {
template hipError_t launch_select_shape<4, 4, 2, false>(const SelectArgs&, int,
                                                              hipStream_t);
}  // namespace si
