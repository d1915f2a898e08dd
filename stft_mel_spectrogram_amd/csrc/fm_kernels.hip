// Fused mel-spectrogram forward kernel for gfx950 (MI355X), and its launcher.
//
// One workgroup owns a tile of consecutive frames of one signal and runs the
// whole chain the flashmel 0.1.0 page describes (README "How it works"):
// padded framing as index arithmetic, window, real FFT, |X|^power and the
// sparse mel projection, then writes [B, n_mels, T] with frames contiguous.
//
// Real FFT of N = n_fft points: z[m] = x[2m] + i*x[2m+1] (m < M = N/2) goes
// through a complex M-point FFT, M = N1*N2, in two register passes with one
// LDS exchange between them:
//   pass 1, one thread per (frame, n2):  N1-point DFT over n1 of
//           z[N2*n1 + n2], times exp(-2*pi*i*n2*k1/M), stored Y[f][k1][n2];
//   pass 2, one thread per (frame, pair of k1): N2-point DFTs of Y[f][k1][.]
//           for k1 and N1-k1, giving Z[k1 + N1*k2] and the mirrored bins
//           Z[M - k] in the same thread, so the split into the real spectrum
//              X[k] = (Z[k] + conj Z[M-k]) - i W_N^k (Z[k] - conj Z[M-k])
//           (window pre-scaled by 1/2) and |X|^p need no further exchange.
// The power tile P[f][k] (odd row stride n_fft/2+1) reuses the exchange
// buffer.  The mel projection walks each filter's CSR run only.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fm_dft.h"
#include "fm_internal.h"

namespace fm {

namespace {

struct KArgs {
  const void* in;
  float* out;
  const float2* win2;   // [M]  0.5*(w[2m], w[2m+1])
  const float2* tw_m;   // [M]  exp(-2 pi i j / M)
  const float2* tw_n;   // [M]  exp(-2 pi i k / N)
  const MelRow* rows;   // [n_mels]
  const float* mel_w;   // [nnz]
  long long length;     // samples per signal
  int n_frames;         // frames per signal
  int hop;
  int pad;              // left padding (n_fft/2 with centring, else 0)
  int n_mels;
  int nnz;
  int tile;             // frames per workgroup
  int tiles_per_signal;
  int pad_mode;
  int power_mode;       // 0: |X|^2, 1: |X|, 2: |X|^power
  float half_power;     // power / 2
  int vec_ok;           // interior tiles may use paired (2-sample) loads
  int lds_y_bytes;
};

template <typename T>
__device__ __forceinline__ float sample_to_float(T v);
template <>
__device__ __forceinline__ float sample_to_float<float>(float v) { return v; }
template <>
__device__ __forceinline__ float sample_to_float<int16_t>(int16_t v) {
  return static_cast<float>(v) * (1.0f / 32768.0f);  // exact
}

// Value of the padded signal at position i (i relative to sample 0).
template <typename T>
__device__ __forceinline__ float padded_sample(const T* x, long long i, long long L, int mode) {
  if (i < 0 || i >= L) {
    switch (mode) {
      case FM_PAD_CONSTANT:
        return 0.0f;
      case FM_PAD_REPLICATE:
        i = i < 0 ? 0 : L - 1;
        break;
      case FM_PAD_CIRCULAR:
        i %= L;
        if (i < 0) i += L;
        break;
      default:  // reflect, single reflection (pad < L checked on the host)
        i = i < 0 ? -i : 2 * (L - 1) - i;
        break;
    }
  }
  return sample_to_float<T>(x[i]);
}

// Two consecutive samples starting at an even position of an interior frame.
__device__ __forceinline__ float2 load_pair(const float* x, long long i) {
  return *reinterpret_cast<const float2*>(x + i);
}
__device__ __forceinline__ float2 load_pair(const int16_t* x, long long i) {
  const short2 v = *reinterpret_cast<const short2*>(x + i);
  return make_float2(static_cast<float>(v.x) * (1.0f / 32768.0f),
                     static_cast<float>(v.y) * (1.0f / 32768.0f));
}

__device__ __forceinline__ float power_of(float sq, int mode, float half_power) {
  if (mode == 0) return sq;
  if (mode == 1) return sqrtf(sq);
  return powf(sq, half_power);
}

// Real-spectrum split for the bin pair (k, M-k) and their powers.
__device__ __forceinline__ void split_pair(float* prow, int k, int kmirror, float2 zk, float2 zm,
                                           float2 w, int mode, float hp) {
  const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);  // Z[k] + conj Z[M-k]
  const float2 o = make_float2(zk.x - zm.x, zk.y + zm.y);  // Z[k] - conj Z[M-k]
  const float2 v = cmul(w, o);
  const float ax = e.x + v.y, ay = e.y - v.x;  // X[k]   = e - i v
  const float bx = e.x - v.y, by = e.y + v.x;  // X[M-k] = conj(e + i v)
  prow[k] = power_of(fmaf(ax, ax, ay * ay), mode, hp);
  prow[kmirror] = power_of(fmaf(bx, bx, by * by), mode, hp);
}

template <int N1, int N2, typename InT>
__global__ __launch_bounds__(256) void mel_forward_kernel(KArgs a) {
  constexpr int M = N1 * N2;
  constexpr int K = M + 1;       // one-sided bins; odd, so P rows are bank-skewed
  constexpr int NF = 2 * M;      // n_fft
  constexpr int NPAIR = N1 / 2;  // pass-2 threads per frame
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);
  float* P = reinterpret_cast<float*>(lds);
  float* Wm = reinterpret_cast<float*>(lds + a.lds_y_bytes);
  MelRow* rows = reinterpret_cast<MelRow*>(Wm + ((a.nnz + 3) & ~3));

  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.tiles_per_signal;
  const int t0 = (blockIdx.x - b * a.tiles_per_signal) * a.tile;
  const int nvalid = min(a.tile, a.n_frames - t0);
  const long long L = a.length;
  const InT* x = static_cast<const InT*>(a.in) + static_cast<long long>(b) * L;

  for (int i = tid; i < a.nnz; i += blockDim.x) Wm[i] = a.mel_w[i];
  for (int i = tid; i < a.n_mels; i += blockDim.x) rows[i] = a.rows[i];

  const long long s_first = static_cast<long long>(t0) * a.hop - a.pad;
  const long long s_last = static_cast<long long>(t0 + nvalid - 1) * a.hop - a.pad + NF - 1;
  const bool interior = a.vec_ok && s_first >= 0 && s_last < L;

  // ---- pass 1: window + N1-point DFTs, twiddle, exchange through LDS ------
  for (int job = tid; job < a.tile * N2; job += blockDim.x) {
    const int f = job / N2;
    const int n2 = job - f * N2;
    if (f >= nvalid) break;
    const long long base = static_cast<long long>(t0 + f) * a.hop - a.pad;
    float2 v[N1];
    if (interior) {
#pragma unroll
      for (int n1 = 0; n1 < N1; ++n1) {
        const int m = N2 * n1 + n2;
        const float2 s = load_pair(x, base + 2 * m);
        const float2 w = a.win2[m];
        v[n1] = make_float2(s.x * w.x, s.y * w.y);
      }
    } else {
#pragma unroll
      for (int n1 = 0; n1 < N1; ++n1) {
        const int m = N2 * n1 + n2;
        const float2 w = a.win2[m];
        v[n1] = make_float2(padded_sample(x, base + 2 * m, L, a.pad_mode) * w.x,
                            padded_sample(x, base + 2 * m + 1, L, a.pad_mode) * w.y);
      }
    }
    Dft<N1>::run(v);
    float2* yrow = Y + (f * N1) * N2 + n2;
    yrow[0] = v[0];
#pragma unroll
    for (int k1 = 1; k1 < N1; ++k1) yrow[k1 * N2] = cmul(v[k1], a.tw_m[n2 * k1]);
  }
  __syncthreads();

  // ---- pass 2: paired N2-point DFTs, real split, power -> P (aliases Y) ----
  const int f2 = tid / NPAIR;
  const int p = tid - f2 * NPAIR;
  const bool has = tid < a.tile * NPAIR && f2 < nvalid;
  float2 za[N2], zb[N2];
  if (has) {
    const int ka = p;
    const int kb = (p == 0) ? N1 / 2 : N1 - p;
    const float2* ra = Y + (f2 * N1 + ka) * N2;
    const float2* rb = Y + (f2 * N1 + kb) * N2;
#pragma unroll
    for (int n2 = 0; n2 < N2; ++n2) {
      za[n2] = ra[n2];
      zb[n2] = rb[n2];
    }
    Dft<N2>::run(za);
    Dft<N2>::run(zb);
  }
  __syncthreads();
  if (has) {
    float* prow = P + f2 * K;
    const int mode = a.power_mode;
    const float hp = a.half_power;
    if (p != 0) {
      // bins k = p + N1*k2 (from za) and M - k = (N1 - p) + N1*(N2-1-k2) (from zb)
#pragma unroll
      for (int k2 = 0; k2 < N2; ++k2) {
        const int k = p + N1 * k2;
        split_pair(prow, k, M - k, za[k2], zb[N2 - 1 - k2], a.tw_n[k], mode, hp);
      }
    } else {
      // k1 = 0: bins N1*k2 pair with N1*(N2-k2) inside za
#pragma unroll
      for (int k2 = 0; k2 <= N2 / 2; ++k2) {
        const int k = N1 * k2;
        split_pair(prow, k, M - k, za[k2], za[(N2 - k2) % N2], a.tw_n[k], mode, hp);
      }
      // k1 = N1/2: bins N1/2 + N1*k2 pair with N1/2 + N1*(N2-1-k2) inside zb
#pragma unroll
      for (int k2 = 0; k2 <= (N2 - 1) / 2; ++k2) {
        const int k = N1 / 2 + N1 * k2;
        split_pair(prow, k, M - k, zb[k2], zb[N2 - 1 - k2], a.tw_n[k], mode, hp);
      }
    }
  }
  __syncthreads();

  // ---- mel projection over each filter's CSR run, frames-contiguous store ---
  const int G = a.tile;
  for (int job = tid; job < a.n_mels * G; job += blockDim.x) {
    const int m = job / G;
    const int f = job - m * G;
    if (f >= nvalid) continue;
    const MelRow r = rows[m];
    const float* pr = P + f * K + r.first;
    const float* wr = Wm + r.off;
    float acc = 0.0f;
    for (int j = 0; j < r.len; ++j) acc = fmaf(wr[j], pr[j], acc);
    a.out[(static_cast<long long>(b) * a.n_mels + m) * a.n_frames + t0 + f] = acc;
  }
}

template <int N1, int N2>
void* kernel_for(int in_dtype) {
  if (in_dtype == FM_I16) return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, int16_t>);
  return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, float>);
}

void* select_kernel(const Plan& p, int in_dtype) {
  if (p.fft.n1 == 8 && p.fft.n2 == 25) return kernel_for<8, 25>(in_dtype);
  if (p.fft.n1 == 32 && p.fft.n2 == 16) return kernel_for<32, 16>(in_dtype);
  if (p.fft.n1 == 32 && p.fft.n2 == 32) return kernel_for<32, 32>(in_dtype);
  return nullptr;
}

int hip_fail(hipError_t e, const char* what) {
  std::string msg = std::string(what) + ": " + hipGetErrorString(e);
  return set_error(FM_E_HIP, msg);
}

}  // namespace

int upload_plan(Plan& p) {
  hipError_t e = hipGetDevice(&p.device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const int M = p.n_fft / 2;
  // one block: win2 | tw_m | tw_n | rows | mel_w, each 256-byte aligned
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const size_t o_win = 0;
  const size_t o_twm = o_win + al(M * sizeof(float2));
  const size_t o_twn = o_twm + al(M * sizeof(float2));
  const size_t o_rows = o_twn + al(M * sizeof(float2));
  const size_t o_w = o_rows + al(p.n_mels * sizeof(MelRow));
  const size_t total = o_w + al(static_cast<size_t>(p.nnz > 0 ? p.nnz : 1) * sizeof(float));
  std::vector<unsigned char> host(total, 0);
  float* win2 = reinterpret_cast<float*>(host.data() + o_win);
  for (int j = 0; j < p.n_fft; ++j) win2[j] = 0.5f * p.window[j];  // exact scaling
  std::copy(p.tw_m.begin(), p.tw_m.end(), reinterpret_cast<float*>(host.data() + o_twm));
  std::copy(p.tw_n.begin(), p.tw_n.end(), reinterpret_cast<float*>(host.data() + o_twn));
  std::copy(p.rows.begin(), p.rows.end(), reinterpret_cast<MelRow*>(host.data() + o_rows));
  std::copy(p.mel_w.begin(), p.mel_w.end(), reinterpret_cast<float*>(host.data() + o_w));
  void* d = nullptr;
  e = hipMalloc(&d, total);
  if (e != hipSuccess) return set_error(FM_E_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
  e = hipMemcpy(d, host.data(), total, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(d);
    return hip_fail(e, "hipMemcpy (plan tables)");
  }
  unsigned char* base = static_cast<unsigned char*>(d);
  p.d_block = d;
  p.d_win2 = base + o_win;
  p.d_tw_m = base + o_twm;
  p.d_tw_n = base + o_twn;
  p.d_rows = base + o_rows;
  p.d_mel_w = base + o_w;
  // Tiles above 64 KB of LDS need the per-kernel opt-in.
  for (int dt : {FM_F32, FM_I16}) {
    void* k = select_kernel(p, dt);
    if (!k) return set_error(FM_E_UNSUPPORTED, "no kernel for this n_fft");
    e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
  }
  p.has_device = true;
  return FM_OK;
}

void free_plan_device(Plan& p) {
  if (p.d_block) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p.device) (void)hipSetDevice(p.device);
    (void)hipFree(p.d_block);
    if (cur != p.device && cur >= 0) (void)hipSetDevice(cur);
  }
  p.d_block = nullptr;
  p.has_device = false;
}

int launch_forward(const Plan& p, const void* in, int in_dtype, int64_t batch, int64_t length,
                   float* out, void* stream) {
  if (!p.has_device) return set_error(FM_E_NODEVICE, "plan was built without device tables");
  if (in_dtype != FM_F32 && in_dtype != FM_I16) return set_error(FM_E_INVAL, "in_dtype must be FM_F32 or FM_I16");
  if (batch < 0) return set_error(FM_E_INVAL, "batch must be >= 0");
  const int64_t T = out_frames(p, length);
  if (T < 0) return static_cast<int>(T);
  if (batch == 0) return FM_OK;
  if (!in || !out) return set_error(FM_E_INVAL, "null input or output pointer");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != p.device) return set_error(FM_E_INVAL, "plan belongs to another device than the current one");
  const int64_t tiles = (T + p.tile_frames - 1) / p.tile_frames;
  if (T > INT32_MAX || tiles * batch > INT32_MAX) return set_error(FM_E_INVAL, "problem too large for one launch");

  KArgs a;
  a.in = in;
  a.out = out;
  a.win2 = static_cast<const float2*>(p.d_win2);
  a.tw_m = static_cast<const float2*>(p.d_tw_m);
  a.tw_n = static_cast<const float2*>(p.d_tw_n);
  a.rows = static_cast<const MelRow*>(p.d_rows);
  a.mel_w = static_cast<const float*>(p.d_mel_w);
  a.length = length;
  a.n_frames = static_cast<int>(T);
  a.hop = p.hop;
  a.pad = p.pad_left;
  a.n_mels = p.n_mels;
  a.nnz = p.nnz;
  a.tile = p.tile_frames;
  a.tiles_per_signal = static_cast<int>(tiles);
  a.pad_mode = p.pad_mode;
  a.power_mode = (p.power == 2.0) ? 0 : (p.power == 1.0 ? 1 : 2);
  a.half_power = static_cast<float>(p.power * 0.5);
  const size_t esz = (in_dtype == FM_I16) ? 2 : 4;
  const uintptr_t ia = reinterpret_cast<uintptr_t>(in);
  a.vec_ok = (ia % (2 * esz) == 0) && (length % 2 == 0) && (p.hop % 2 == 0) && (p.pad_left % 2 == 0);
  a.lds_y_bytes = p.lds_y_bytes;

  void* k = select_kernel(p, in_dtype);
  if (!k) return set_error(FM_E_UNSUPPORTED, "no kernel for this n_fft");
  void* args[] = {&a};
  e = hipLaunchKernel(k, dim3(static_cast<unsigned>(tiles * batch)), dim3(p.threads), args,
                      static_cast<size_t>(p.lds_bytes), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return FM_OK;
}

}  // namespace fm
