// Paired forward kernels for n_fft = 400: complex FFT of 400 = 20 x 20 points.
#include "fm_pair.h"

namespace fm {
template void* pair_kernel_for<20>(int, int);
}  // namespace fm
