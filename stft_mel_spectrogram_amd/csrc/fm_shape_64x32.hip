// Kernels for n_fft = 4096: complex FFT of 2048 = 64 x 32 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<64, 32>(int, int, bool, bool, bool);
template void* backward_kernel_for<64, 32>(int);
}  // namespace fm
