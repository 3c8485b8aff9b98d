// Two-pass RMSNorm kernels for rows of 7168, 8192 columns or fewer (superchunk
// counts 7, 8).
#include "rows.hpp"

namespace nvfp4q {

template void launch_rms_nsc<7>(const RowArgs&, bool, hipStream_t);
template void launch_rms_nsc<8>(const RowArgs&, bool, hipStream_t);

}  // namespace nvfp4q
