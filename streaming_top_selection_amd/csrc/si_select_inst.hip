// One explicit instantiation of the select kernel per (register-tile shape, operand
// mode): the build compiles this file once per pair with SI_NW, SI_KB, SI_NS (waves,
// key blocks per wave, register tiles per key tile) and SI_OP defined, so the kernels
// compile in parallel.
#include "si_select.hpp"

#if !defined(SI_NW) || !defined(SI_KB) || !defined(SI_NS) || !defined(SI_OP)
#error "si_select_inst.hip is compiled with -DSI_NW=.. -DSI_KB=.. -DSI_NS=.. -DSI_OP=.."
#endif

namespace si {
template hipError_t launch_select_shape<SI_NW, SI_KB, SI_NS, SI_OP>(const SelectArgs&, int,
                                                                    hipStream_t);
}  // namespace si
