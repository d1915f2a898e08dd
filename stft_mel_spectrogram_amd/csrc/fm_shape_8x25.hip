// Kernels for n_fft = 400: complex FFT of 200 = 8 x 25 points.
#include "fm_kernel.h"

namespace fm {
template void* kernel_for<8, 25>(int, int, bool);
}  // namespace fm
