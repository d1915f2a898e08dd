// Internal declarations shared by the host plan builder, the C ABI and the
// HIP kernels of the fused mel-spectrogram forward pass.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "fm.h"

namespace fm {

// Per-mel CSR row: first bin of the contiguous support, number of bins,
// offset of its first weight in the packed weight array.
struct MelRow {
  int32_t first, len, off, pad_;
};

// One step of a wave's sweep over consecutive bins in the mel stage: the
// weights of the bin in the (at most two) filters open at that bin, and the
// filters that end at it.  code = n_end | (mel_a << 8) | (mel_b << 16): after
// the bin, n_end (0..2) open filters end, the older one being mel_a.
struct SweepStep {
  float wa, wb;
  int32_t code, pad_;
};

// A wave's share of the mel stage: bins k0 .. k0 + nsteps - 1 (nsteps a
// multiple of 8, tail steps zero), and the empty filters it writes as 0.
struct WaveSweep {
  int32_t k0, step_off, nsteps, empty_off, n_empty;
};

// FFT factorisation of the complex transform of n_fft/2 points that carries
// the real FFT (even samples as real part, odd samples as imaginary part).
struct FftShape {
  int n1, n2;  // n_fft/2 = n1 * n2
};

struct Plan {
  // transform arguments
  int sample_rate = 0, n_fft = 0, win_length = 0, hop = 0, n_mels = 0;
  double f_min = 0, f_max = 0, power = 2.0;
  int center = 1, pad_mode = FM_PAD_REFLECT, mel_scale = FM_MEL_HTK, norm = FM_NORM_NONE;
  // derived
  int n_freqs = 0;     // n_fft/2 + 1
  int pad_left = 0;    // samples of centre padding on each side
  FftShape fft{0, 0};
  int tile_max = 0;      // most frames a workgroup tile may hold
  int tile_override = 0; // FM_TILE_FRAMES, for sweeps (0: chosen per call)
  int threads = 256;
  int lds_bytes = 0;     // dynamic LDS of a tile of tile_max frames
  int mel_split[5] = {0, 0, 0, 0, 0};  // mel rows of each of the 4 waves
  WaveSweep sweep[4] = {};             // per-wave mel sweep
  std::vector<SweepStep> steps;        // all waves' sweep steps
  std::vector<int32_t> empty_mels;     // filters with no bin, by wave
  int nnz = 0, w_max = 0;
  // host tables (float32 after one rounding from float64)
  std::vector<float> window;  // [n_fft], unscaled
  std::vector<MelRow> rows;   // [n_mels]
  std::vector<float> mel_w;   // [nnz]
  std::vector<float> tw_m;    // [2*M] exp(-2 pi i j / M), M = n_fft/2
  std::vector<float> tw_n;    // [2*M] exp(-2 pi i k / n_fft)
  // device
  bool has_device = false;
  int device = -1;
  int n_cu = 0;                // compute units of that device
  void* d_block = nullptr;     // one allocation holding every table
  const void* d_win2 = nullptr;   // float2[M] : 0.5*(w[2m], w[2m+1])
  const void* d_tw_m = nullptr;   // float2[M]
  const void* d_tw_n = nullptr;   // float2[M]
  const void* d_rows = nullptr;   // MelRow[n_mels]
  const void* d_mel_w = nullptr;  // float[nnz]
  const void* d_steps = nullptr;  // SweepStep[steps.size()]
  const void* d_empty = nullptr;  // int32[empty_mels.size()]
};

// Thread-local error reporting.
int set_error(int code, const std::string& msg);
const char* last_error_cstr();

// Builds every host table and the tile geometry; touches no GPU.
int build_host_plan(Plan& p, int sample_rate, int n_fft, int win_length,
                    int hop_length, int n_mels, double f_min, double f_max,
                    double power, int center, int pad_mode, int mel_scale,
                    int norm);

// Dynamic LDS of a tile of `frames` frames: the exchange / power buffer,
// then the staged mel weights and CSR rows.
int tile_exchange_bytes(const Plan& p, int frames);
int tile_lds_bytes(const Plan& p, int frames);

// Frames per signal for a plan (negative FM_E_* on invalid length).
int64_t out_frames(const Plan& p, int64_t length);

// Device side (fm_kernels.hip).
int upload_plan(Plan& p);
void free_plan_device(Plan& p);
int launch_forward(const Plan& p, const void* in, int in_dtype, int64_t batch,
                   int64_t length, float* out, void* stream);

}  // namespace fm
