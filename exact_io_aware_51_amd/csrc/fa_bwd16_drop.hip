// fa_bwd16_drop.hip -- the dropout instantiations of the 16-bit backward
// kernels (fa_bwd16.hip), compiled as a unit of their own.
//
// The rest of the 16-bit backward is scheduled with LLVM's max-ILP strategy,
// which is faster for it but makes the dropout kernels 17% slower (c5 shape,
// p = 0.1); the scheduling strategy is chosen per compilation unit, so these
// kernels are built here with the default one.  The two units instantiate
// disjoint sets of kernels: fa_bwd16.hip calls launch_dq16_drop /
// launch_dkdv16_drop for dropout and instantiates no dropout kernel itself.
#define FA_BWD16_DROPOUT_UNIT 1
#include "fa_bwd16.hip"
