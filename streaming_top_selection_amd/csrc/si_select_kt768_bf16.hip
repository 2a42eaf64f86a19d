// Select kernels for key tile 768 (4 waves x 2 blocks x 3 register tiles), bf16 keys.
#include "si_select.hpp"

namespace si {
template hipError_t launch_select_shape<4, 2, 3, false>(const SelectArgs&, int,
                                                              hipStream_t);
}  // namespace si
