// fa_fwd16_d128.hip -- the d = 128 instantiations of the 16-bit forward
// kernels (fa_fwd16.hip), compiled as a unit of their own.
//
// They are scheduled with LLVM's max-ILP strategy, which is faster for them
// (c5-shape forward +3-4%, c2 +2%) but makes the d = 64 forward 4% slower;
// the strategy is chosen per compilation unit, so d = 64 stays in
// fa_fwd16.hip with the default.  fa_fwd16.hip calls launch_fwd16_128 for
// d = 128 and instantiates no d = 128 kernel itself.
#define FA_FWD16_D128_UNIT 1
#include "fa_fwd16.hip"
