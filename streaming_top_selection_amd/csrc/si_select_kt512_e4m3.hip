// Select kernels for key tile 512 (4 waves x 4 blocks x 1 register tiles), e4m3 keys.
#include "si_select.hpp"

namespace si {
template hipError_t launch_select_shape<4, 4, 1, true>(const SelectArgs&, int,
                                                              hipStream_t);
}  // namespace si
