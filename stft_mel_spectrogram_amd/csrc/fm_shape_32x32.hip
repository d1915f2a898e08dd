// Kernels for n_fft = 2048: complex FFT of 1024 = 32 x 32 points.
#include "fm_backward.h"

namespace fm {
template void* kernel_for<32, 32>(int, int, bool, bool, bool);
template void* backward_kernel_for<32, 32>(int);
}  // namespace fm
