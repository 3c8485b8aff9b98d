// Two-pass RMSNorm kernels for rows of 1024, 2048, 4096 columns or fewer (superchunk
// counts 1, 2, 4).
#include "rows.hpp"

namespace nvfp4q {

template void launch_rms_nsc<1>(const RowArgs&, bool, hipStream_t);
template void launch_rms_nsc<2>(const RowArgs&, bool, hipStream_t);
template void launch_rms_nsc<4>(const RowArgs&, bool, hipStream_t);

}  // namespace nvfp4q
