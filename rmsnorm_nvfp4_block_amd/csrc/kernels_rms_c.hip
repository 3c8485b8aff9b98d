// Two-pass RMSNorm kernels for rows of 12288, 16384 columns or fewer (superchunk
// counts 12, 16).
#include "rows.hpp"

namespace nvfp4q {

template void launch_rms_nsc<12>(const RowArgs&, bool, hipStream_t);
template void launch_rms_nsc<16>(const RowArgs&, bool, hipStream_t);

}  // namespace nvfp4q
