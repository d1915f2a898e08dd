// Fused mel-spectrogram forward kernel for gfx950 (MI355X): device code.
// Each fm_shape_<n1>x<n2>.hip instantiates it for one FFT shape;
// fm_launch.hip uploads plans and launches it.
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
//   pass 2, in one of two layouts (template flag ROWS, chosen per call):
//           pair layout, one thread per (frame, pair of k1): N2-point DFTs
//           of Y[f][k1][.] for k1 and N1-k1, giving Z[k1 + N1*k2] and the
//           mirrored bins Z[M - k] in the same thread; row layout (512
//           threads), one thread per (frame, k1): one N2-point DFT, the
//           mirrored row's values fetched from the partner lane.  Either way
//           the split into the real spectrum
//              X[k] = (Z[k] + conj Z[M-k]) - i W_N^k (Z[k] - conj Z[M-k])
//           (window pre-scaled by 1/2) and |X|^p follow with the same
//           operations in the same order.
// A tile's samples are gathered per frame or, in the COPY variants, copied
// into LDS as one contiguous span first (also chosen per call).
// The power tile P[f][k] (odd frame stride n_fft/2+1) reuses the exchange
// buffer (rows of N2 complex values, padded to N2 + 1 where N2 is even;
// frames 4 complex values apart beyond their rows).  The mel projection is
// a block-sparse product on the matrix cores: 16 filters x 16 frames per
// v_mfma_f32_16x16x4f32, over only the bins each block of filters touches.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "fm_dft.h"
#include "fm_internal.h"

namespace fm {

// Kernel arguments (one struct, passed by value).
struct KArgs {
  const void* in;
  void* out;            // [B, n_mels, n_frames] float or _Float16
  const float2* win2;   // [M]  0.5*(w[2m], w[2m+1])
  const float2* tw_m;   // [M]  first-pass twiddles exp(-2 pi i n2 k1 / M),
                        //      entry k1*N2 + n2 (consecutive threads, consecutive
                        //      entries)
  const float2* tw_n;   // [M]  exp(-2 pi i k / N)
  long long length;     // samples per signal
  int n_frames;         // frames per signal
  int hop;
  int pad;              // first frame's offset before sample 0: centre padding
                        // (n_fft/2, or 0) + zero padding
  int zpad;             // zero samples added on both sides of the signal
  int n_mels;
  int tile;             // frames per workgroup tile (<= 64)
  int tiles_per_signal;
  int pad_mode;
  float half_power;     // power / 2
  int vec_ok;           // interior tiles may use paired (2-sample) loads
  const int* mel_tbl;   // wave_beg[5], 3 pad, then {kb, step word (mel_step_word), w_off, filter word (mel_filter_word)} per block
  const float* blk_w;   // block weights, 64 per 4-bin step (MFMA A-operand order)
  int w_chunks;         // block weights / 256 (copied to LDS in 1 KB chunks;
                        // 0 when the shape reads them from global memory)
  int w_lds;            // LDS float offset of the copied weights
  int out_f16;          // 1: the output is float16
  int tab_lds;          // LDS byte offset of the pass-1 tables (tables_in_lds)
  int twn_lds;          // LDS byte offset of the split twiddles (n_fft/2 > 256)
  int mel_valu;         // 1: this call's tiles project on the vector units (mel_valu)
  const int* quad_tbl;  // quad_beg[kMelShares + 1], pad to 16, then kQuadHdr int32 per quad
  const float* quad_w;  // quad weights, 4 per step
};

namespace {

// Tables read with wave-uniform indices are reached through the constant
// address space so they load as scalars (SGPR operands of the FMAs).
using CInt = const __attribute__((address_space(4))) int;
using CFloat = const __attribute__((address_space(4))) float;

using f32x4 = float __attribute__((ext_vector_type(4)));

// Mel projection of one wave's blocks on the matrix cores.  Per block of 16
// filters and per 4-bin step, one v_mfma_f32_16x16x4f32 for each 16-frame
// column group (NFB of them):
//   A (16 filters x 4 bins)  weights, lane l: filter l%16, bin l/16;
//   B (4 bins x 16 frames)   power tile, lane l: bin l/16, frame l%16;
//   D (16 x 16)              lane l holds filters 4*(l/16) + r, r < 4, of
//                            frame l%16.
// KS is the power tile's frame stride.  Both operands come from LDS (the
// weights were copied there); blocks are
// padded to whole groups of kMelStepGroup steps, so the step loop has no
// tail.  Columns beyond the last valid frame read that frame again and are
// not stored, so no column reads a power row that was not written; a step
// run may reach up to 15 floats past a row's last bin, into the next row
// (times zero weights) or, after the last valid frame, into floats the
// kernel zeroes.
// Output (element type OT: float, or _Float16 rounded to nearest): with
// STAGE the 16 x 16*NFB result goes through the wave's LDS staging area
// `stg` and each filter row leaves in one contiguous streaming store (lane =
// frame); otherwise lanes store their D elements directly (plain stores, so
// that L2 merges the pieces of a row).
// GW: the weights WL are in global memory (large FFTs); they are loaded
// kMelGlobalChunk steps at a time, then consumed group by group.
template <int KS, int NFB, bool STAGE, bool GW, typename OT>
__device__ __forceinline__ void mel_blocks(const float* P, const float* WL, float* stg, int G,
                                           int nvalid, int lane, OT* obase, int n_frames,
                                           int n_mels, CInt* blk, int bb, int be, int bstep) {
  constexpr int U = kMelStepGroup;
  const int fr = lane & 15, kq = lane >> 4;
  int roff[NFB];
#pragma unroll
  for (int f = 0; f < NFB; ++f) roff[f] = min(16 * f + fr, nvalid - 1) * KS + kq;
  for (int bi = bb; bi < be; bi += bstep) {
    // Step word (mel_step_word): ksteps, and s_hi, from which on every step
    // holds only zero weights.  The wide-tile (STAGE) and global-weight (GW)
    // instantiations stop at s_hi: they skip the groups past it and, in the
    // group holding it, the products of the zero steps (8 x 480000 at n_fft
    // 400: 16.3 against 16.6 us; n_fft 4096, 4 x 1323000: 74.6 against 76.5
    // us).  The others run every padded step: with the branches the
    // narrow-tile loop measured 3-7% slower (n_fft 2048: 97.2 against 91.1).
    constexpr bool kSkip = STAGE || GW;
    const int kb = blk[4 * bi], sw = blk[4 * bi + 1], woff = blk[4 * bi + 2],
              fw = blk[4 * bi + 3];
    const int mel0 = fw & 0xffff, nrow = fw >> 16;  // filters mel0 .. mel0 + nrow - 1 (mel_filter_word)
    const int s_end = kSkip ? sw >> 20 : (sw & 1023);
    f32x4 acc[NFB];
#pragma unroll
    for (int f = 0; f < NFB; ++f) acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float* pb = P + kb;
    const float* wl = WL + woff + lane;
    auto group = [&](const float* av, const float* pg, int nu) {
      float bv[U][NFB];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int f = 0; f < NFB; ++f) bv[u][f] = pg[roff[f] + 4 * u];
      if (!kSkip || nu >= U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int f = 0; f < NFB; ++f)
            acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u][f], acc[f], 0, 0, 0);
      } else {
#pragma unroll
        for (int u = 0; u < U - 1; ++u) {
          if (u < nu) {  // wave-uniform
#pragma unroll
            for (int f = 0; f < NFB; ++f)
              acc[f] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u][f], acc[f], 0, 0, 0);
          }
        }
      }
    };
    if constexpr (GW) {
      constexpr int CH = kMelGlobalChunk;
      for (int s0 = 0; s0 < s_end; s0 += CH, pb += 4 * CH, wl += 64 * CH) {
        float av[CH];  // one chunk of weights in flight at once (slack covers the tail)
#pragma unroll
        for (int j = 0; j < CH; ++j) av[j] = wl[64 * j];
#pragma unroll
        for (int g = 0; g < CH / U; ++g)
          if (s0 + U * g < s_end) group(av + U * g, pb + 4 * U * g, s_end - s0 - U * g);
      }
    } else {
      for (int s0 = 0; s0 < s_end; s0 += U, pb += 4 * U, wl += 64 * U) {
        float av[U];
#pragma unroll
        for (int u = 0; u < U; ++u) av[u] = wl[64 * u];
        group(av, pb, s_end - s0);
      }
    }
    if constexpr (STAGE) {
      constexpr int PITCH = 16 * NFB + 1;  // odd: conflict-free column writes
#pragma unroll
      for (int f = 0; f < NFB; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[(4 * kq + r) * PITCH + 16 * f + fr] = acc[f][r];
      // the rows are read back by other lanes of this wave: LDS operations
      // of one wave complete in order, so waiting for the writes suffices
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      const bool st = lane < nvalid && lane < 16 * NFB;
      const int col = lane < 16 * NFB ? lane : 0;  // lanes past the tile's columns stay in the stage
      for (int m = 0; m < nrow; ++m) {
        const float v = stg[m * PITCH + col];
        // output is written once and never re-read here: streaming stores
        if (st) __builtin_nontemporal_store(static_cast<OT>(v), obase + static_cast<long long>(mel0 + m) * n_frames + lane);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next block's writes
      __builtin_amdgcn_wave_barrier();
    } else {
      const int mrow = mel0 + 4 * kq;
#pragma unroll
      for (int f = 0; f < NFB; ++f) {
        const int frame = 16 * f + fr;
        if (frame < nvalid) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * kq + r < nrow) obase[static_cast<long long>(mrow + r) * n_frames + frame] = static_cast<OT>(acc[f][r]);
        }
      }
    }
  }
}

// Mel projection of a wide tile on the vector units.  Lane l computes frame
// l's outputs (lanes past the last valid frame read that frame's row and
// store nothing).  Each wave walks its quads of 4 consecutive filters: per
// step of a quad the four weights are one scalar load and each filter's
// power value one LDS read, so the quad's four multiply-add chains run side
// by side; a filter's run is padded with zero weights to the quad's length
// and starts early enough to end inside the frame's bins.  Each filter's
// row of the tile then leaves with one streaming store (the tile's frames
// are contiguous in the output).  Against the matrix-core blocks this does
// the filterbank's nonzero products only (n_fft 400, 128 filters: 395 per
// frame, where the 16-filter blocks spend 4096).
template <int KS, typename OT>
__device__ __forceinline__ void mel_valu(const float* P, CInt* qt, CFloat* qw, int nvalid, int lane,
                                         OT* obase, int n_frames, int n_mels, int qb, int qe) {
  const float* prow = P + min(lane, nvalid - 1) * KS;
  const bool st = lane < nvalid;
  for (int q = qb; q < qe; ++q) {
    CInt* h = qt + 16 + kQuadHdr * q;
    const int L = h[4];
    CFloat* w = qw + 4 * h[5];
    const float* p0 = prow + h[0];
    const float* p1 = prow + h[1];
    const float* p2 = prow + h[2];
    const float* p3 = prow + h[3];
    float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
    // four steps per round from running pointers, so that a round's reads
    // share one address per filter (immediate LDS offsets) and its 16
    // weights are one scalar load; then the last 0-3 steps as a pair and a
    // single, straight-line
    int i = 0;
    for (; i + 4 <= L; i += 4, p0 += 4, p1 += 4, p2 += 4, p3 += 4, w += 16) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a0 = fmaf(w[4 * u + 0], p0[u], a0);
        a1 = fmaf(w[4 * u + 1], p1[u], a1);
        a2 = fmaf(w[4 * u + 2], p2[u], a2);
        a3 = fmaf(w[4 * u + 3], p3[u], a3);
      }
    }
    if (L - i >= 2) {
      a0 = fmaf(w[0], p0[0], a0);
      a1 = fmaf(w[1], p1[0], a1);
      a2 = fmaf(w[2], p2[0], a2);
      a3 = fmaf(w[3], p3[0], a3);
      a0 = fmaf(w[4], p0[1], a0);
      a1 = fmaf(w[5], p1[1], a1);
      a2 = fmaf(w[6], p2[1], a2);
      a3 = fmaf(w[7], p3[1], a3);
      i += 2, p0 += 2, p1 += 2, p2 += 2, p3 += 2, w += 8;
    }
    if (L - i >= 1) {
      a0 = fmaf(w[0], p0[0], a0);
      a1 = fmaf(w[1], p1[0], a1);
      a2 = fmaf(w[2], p2[0], a2);
      a3 = fmaf(w[3], p3[0], a3);
    }
    if (st) {
      const int m = 4 * q;  // < n_mels
      OT* o = obase + static_cast<long long>(m) * n_frames + lane;
      __builtin_nontemporal_store(static_cast<OT>(a0), o);
      if (m + 1 < n_mels) __builtin_nontemporal_store(static_cast<OT>(a1), o + n_frames);
      if (m + 2 < n_mels) __builtin_nontemporal_store(static_cast<OT>(a2), o + 2 * n_frames);
      if (m + 3 < n_mels) __builtin_nontemporal_store(static_cast<OT>(a3), o + 3 * n_frames);
    }
  }
}

// Source index of position i of the centre-padded signal (i relative to
// sample 0 of a signal of L samples), or -1 for a constant-zero position.
// The host guarantees that frames reach at most one signal length beyond
// either end, so one reflection or wrap suffices; all indices fit in 32 bits.
__device__ __forceinline__ int padded_index(int i, int L, int mode) {
  if (static_cast<unsigned>(i) < static_cast<unsigned>(L)) return i;
  switch (mode) {
    case FM_PAD_CONSTANT: return -1;
    case FM_PAD_REPLICATE: return i < 0 ? 0 : L - 1;
    case FM_PAD_CIRCULAR: return i < 0 ? i + L : i - L;
    default: return i < 0 ? -i : 2 * (L - 1) - i;  // reflect
  }
}

// Two consecutive samples starting at an even position of an interior frame.
__device__ __forceinline__ float2 load_pair(const float* x, int i) {
  return *reinterpret_cast<const float2*>(x + i);
}
// int16 pairs come back unscaled: the 2^-15 PCM scale is folded into the
// (register-held) window, which keeps the product exact.
__device__ __forceinline__ float2 load_pair_raw(const float* x, int i) { return load_pair(x, i); }
__device__ __forceinline__ float2 load_pair_raw(const int16_t* x, int i) {
  const short2 v = *reinterpret_cast<const short2*>(x + i);
  return make_float2(static_cast<float>(v.x), static_cast<float>(v.y));
}
// Sample at position i (relative to x[0]) of the signal first extended by
// zpad zeros on both sides, then centre-padded in `mode` (the centre padding
// reflects, repeats or wraps the zero-extended signal).
template <typename T>
__device__ __forceinline__ float padded_sample_raw(const T* x, int i, int L, int zpad, int mode) {
  const int e = padded_index(i + zpad, L + 2 * zpad, mode);
  const int j = e - zpad;
  if (e < 0 || static_cast<unsigned>(j) >= static_cast<unsigned>(L)) return 0.0f;
  if constexpr (std::is_same<T, int16_t>::value) return static_cast<float>(x[j]);
  else return x[j];
}
// The same sample in the input's own type (int16 unscaled), 0 at a
// constant-zero position.
template <typename T>
__device__ __forceinline__ T padded_value(const T* x, int i, int L, int zpad, int mode) {
  const int e = padded_index(i + zpad, L + 2 * zpad, mode);
  const int j = e - zpad;
  if (e < 0 || static_cast<unsigned>(j) >= static_cast<unsigned>(L)) return T(0);
  return x[j];
}
// Two consecutive samples from the LDS copy of a tile (int16 unscaled).
template <typename T>
__device__ __forceinline__ float2 lds_pair_raw(const unsigned char* p);
template <>
__device__ __forceinline__ float2 lds_pair_raw<float>(const unsigned char* p) {
  return *reinterpret_cast<const float2*>(p);
}
template <>
__device__ __forceinline__ float2 lds_pair_raw<int16_t>(const unsigned char* p) {
  const short2 v = *reinterpret_cast<const short2*>(p);
  return make_float2(static_cast<float>(v.x), static_cast<float>(v.y));
}

template <typename T>
constexpr float kSampleScale = std::is_same<T, int16_t>::value ? (1.0f / 32768.0f) : 1.0f;

// Workgroup -> tile order.  The dispatcher deals workgroups to the chip's 8
// XCDs in turn (workgroup i to XCD i mod 8), and each XCD has its own L2:
// tile i + 1 on another XCD than tile i would fetch the 128-byte lines the
// two tiles share (input halo, output rows where tiles meet) a second time.
// This order gives XCD x the contiguous tiles [x*q + min(x, r), ...) of n
// = 8q + r, so neighbouring tiles share an L2 (a bijection on [0, n)).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile_order(int wg, int n) {
  const int q = n / kXcds, r = n - q * kXcds;
  const int x = wg % kXcds, i = wg / kXcds;
  return x * q + min(x, r) + i;
}

// |X|^p from |X|^2: PMODE 0 -> p = 2, 1 -> p = 1, 2 -> any p > 0 (hp = p/2).
template <int PMODE>
__device__ __forceinline__ float power_of(float sq, float hp) {
  if constexpr (PMODE == 0) {
    return sq;
  } else if constexpr (PMODE == 1) {
    return __builtin_amdgcn_sqrtf(sq);  // v_sqrt_f32, within 1 ulp
  } else {
    // |X|^p = 2^(p/2 * log2 |X|^2) with v_log_f32 / v_exp_f32 (1 ulp each)
    return sq > 0.0f ? __builtin_amdgcn_exp2f(hp * __builtin_amdgcn_logf(sq)) : 0.0f;
  }
}

// Real-spectrum split for the bin pair (k, M-k): powers to *pk and *pm.
template <int PMODE>
__device__ __forceinline__ void split_pair(float* pk, float* pm, float2 zk, float2 zm, float2 w,
                                           float hp) {
  const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);  // Z[k] + conj Z[M-k]
  const float2 o = make_float2(zk.x - zm.x, zk.y + zm.y);  // Z[k] - conj Z[M-k]
  const float2 v = cmul(w, o);
  const float ax = e.x + v.y, ay = e.y - v.x;  // X[k]   = e - i v
  const float bx = e.x - v.y, by = e.y + v.x;  // X[M-k] = conj(e + i v)
  *pk = power_of<PMODE>(fmaf(ax, ax, ay * ay), hp);
  *pm = power_of<PMODE>(fmaf(bx, bx, by * by), hp);
}

// Pair layout: two waves per SIMD (<= 256 registers each): two workgroups
// per compute unit wherever two tiles fit the LDS, or one workgroup of 8
// waves (n_fft = 2048, whose tile takes the whole LDS); n_fft = 4096 runs one
// wave per SIMD.  Row layout (ROWS): 8 waves, four per SIMD (<= 128
// registers: two tiles per CU) where the second pass's rows are short, else
// two per SIMD.
template <int N1, int N2, bool ROWS>
constexpr int kMinWavesPerSimd = ROWS ? rows_waves_per_simd(N1, N2) : ((N1 * N2 <= 1024) ? 2 : 1);
template <int N1, int N2, bool ROWS>
constexpr int kThreads = ROWS ? kRowsThreads : threads_for(N1, N2);

// Shapes that can copy a tile's samples into LDS first (COPY variant,
// chosen per call; copy_capable in fm_internal.h).
template <int N1, int N2>
constexpr bool kCopyCapable = copy_capable(N1, N2);
// The row layout is built up to N1 = 32: at N1 = 64 its 512 threads leave
// each wave 256 registers, which the 64-point first pass overflows.
template <int N1, int N2>
constexpr bool kRowsCapable = N1 <= kRowsMaxN1;

// PRIO: the waves lower their issue priority phase by phase (pass 1
// highest, the mel stage lowest), so that of two workgroups sharing a CU the
// one that is behind issues first (chosen per call, choose_forward).
template <int N1, int N2, typename InT, int PMODE, bool COPY, bool ROWS, bool PRIO>
__global__ __launch_bounds__((kThreads<N1, N2, ROWS>), (kMinWavesPerSimd<N1, N2, ROWS>)) void mel_forward_kernel(KArgs a) {
  constexpr int M = N1 * N2;
  constexpr int K = M + 1;        // one-sided bins
  constexpr int RS = exchange_row(N2);         // LDS row and frame strides (padded)
  constexpr int SY = exchange_stride(N1, N2);
  constexpr int SP = power_stride(M);
  constexpr int NF = 2 * M;       // n_fft
  constexpr int NPAIR = N1 / 2;   // pass-2 threads per frame (pair layout)
  constexpr int NT = kThreads<N1, N2, ROWS>;  // threads of the workgroup
  constexpr int NW = NT / 64;           // waves
  constexpr int SLOTS = NT / N2;  // frames per pass-1 round (one thread per n2)
  constexpr bool kHoist = N1 <= 8;   // window and twiddles in registers, all of
                                     // a thread's samples loaded before compute
  constexpr bool kTabLds = tables_in_lds(N1, M);  // !kHoist: pass-1 tables copied into
                                                  // LDS (else read per frame from L2)
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);  // Y[f][k1][n2]
  float* P = reinterpret_cast<float*>(lds);    // P[f][k], aliases Y
  // pass-1 tables copied behind Y (kTabLds): window pairs, then twiddles
  // (both in the order of KArgs)
  const float2* tab_win = reinterpret_cast<const float2*>(lds + a.tab_lds);
  const float2* tab_tw = tab_win + M;

  const int tid = threadIdx.x;
  const int G = a.tile;
  const int L = static_cast<int>(a.length);

  // pass-1 role of this thread: fixed n2, frames slot, slot+SLOTS, ...
  const int n2 = tid % N2;
  const int slot = tid / N2;
  // pass-2 role: frame f2, and pair p of first-pass output rows (row p
  // itself in the row layout)
  const int f2 = ROWS ? tid / N1 : tid / NPAIR;
  const int p = ROWS ? tid - f2 * N1 : tid - f2 * NPAIR;
  // mel role: wave -> its list of filter blocks
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // Split twiddles W_N^k: for FFTs of up to 256 points each pass-2 thread
  // holds its own in registers; from 1024 points they are copied into LDS
  // at the start (direct global -> LDS loads of 1 KB per wave instruction,
  // behind every other use of the tile's LDS) and read there in the split;
  // the 512-point FFT reads them from L2.  (Measured against reading them
  // from L2, same box: n_fft 2048 115.1 -> 112.7 us, n_fft 4096 98.9 ->
  // 98.5 us, n_fft 1024 13.7 -> 14.0 us.)
  constexpr bool kTwPrefetch = M <= 256;
  constexpr bool kTwLds = twiddles_in_lds(M);
  const float2* twn_l = reinterpret_cast<const float2*>(lds + a.twn_lds);
  if constexpr (kTwLds) {
    static_assert(M % 128 == 0, "whole 1 KB chunks of twiddles");
    for (int c = wave; c < M / 128; c += NW)
      __builtin_amdgcn_global_load_lds(a.tw_n + c * 128 + lane * 2, lds + a.twn_lds + c * 1024, 16, 0, 0);
  }

  // One tile per workgroup.  (Looping over tiles would let the compiler hoist
  // the per-thread table loads out of the loop and keep them live across
  // every pass, which costs more registers than it saves.)
  {
    const int tile = __builtin_amdgcn_readfirstlane(xcd_tile_order(blockIdx.x, gridDim.x));
    const int b = tile / a.tiles_per_signal;
    const int t0 = (tile - b * a.tiles_per_signal) * G;
    const int nvalid = min(G, a.n_frames - t0);
    const InT* x = static_cast<const InT*>(a.in) + static_cast<long long>(b) * L;

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(3);  // pass 1
    // ---- pass 1: window + N1-point DFTs, twiddle, exchange through LDS ----
    const bool p1 = slot < SLOTS;  // threads with a pass-1 role
    {
      float2 win[kHoist ? N1 : 1], twv[kHoist ? N1 : 1];
      if constexpr (kHoist) {
#pragma unroll
        for (int n1 = 0; n1 < N1; ++n1) win[n1] = a.win2[N2 * n1 + n2];
        if constexpr (!std::is_same<InT, float>::value) {
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1)
            win[n1] = make_float2(win[n1].x * kSampleScale<InT>, win[n1].y * kSampleScale<InT>);
        }
        twv[0] = make_float2(1.0f, 0.0f);
#pragma unroll
        for (int k1 = 1; k1 < N1; ++k1) twv[k1] = a.tw_m[N2 * k1 + n2];
      }
      auto fetch = [&](int f, float2 (&s)[N1]) {
        const int base = (t0 + f) * a.hop - a.pad;
        if (a.vec_ok && base >= 0 && base + NF <= L) {  // interior frame
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1) s[n1] = load_pair_raw(x, base + 2 * (N2 * n1 + n2));
        } else {
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1) {
            const int i = base + 2 * (N2 * n1 + n2);
            s[n1] = make_float2(padded_sample_raw(x, i, L, a.zpad, a.pad_mode),
                                padded_sample_raw(x, i + 1, L, a.zpad, a.pad_mode));
          }
        }
      };
      auto compute = [&](int f, const float2 (&s)[N1]) {
        float2 v[N1];
#pragma unroll
        for (int n1 = 0; n1 < N1; ++n1) {
          float2 w;
          if constexpr (kHoist) {
            w = win[kHoist ? n1 : 0];  // already scaled for int16
          } else {
            w = kTabLds ? tab_win[N2 * n1 + n2] : a.win2[N2 * n1 + n2];
            w = make_float2(w.x * kSampleScale<InT>, w.y * kSampleScale<InT>);
          }
          v[n1] = make_float2(s[n1].x * w.x, s[n1].y * w.y);
        }
        Dft<N1>::run(v);
        float2* yrow = Y + f * SY + n2;
        yrow[0] = v[0];
#pragma unroll
        for (int k1 = 1; k1 < N1; ++k1)
          yrow[k1 * RS] = cmul(v[k1], kHoist ? twv[kHoist ? k1 : 0]
                                             : (kTabLds ? tab_tw[N2 * k1 + n2] : a.tw_m[N2 * k1 + n2]));
      };
      // Whole-tile sample copy (COPY variants): the tile's contiguous span
      // of samples is copied into LDS first, with 16-byte direct loads (a
      // few wide instructions per wave instead of one 8-byte gather per
      // sample pair, and each sample read once instead of n_fft/hop times).
      // The loads take the 16-byte chunks that lie inside the signal; the
      // span's other positions (the padding at a signal's ends, and the
      // partial chunks next to them) are filled one sample each through the
      // padding index map, so edge tiles copy too.  The copy aliases the
      // exchange buffer, so every thread takes its samples into registers
      // before the first Y store.  Returns the LDS address of the tile's
      // first (padded) sample once the copy is complete, or null where the
      // input is not aligned for paired reads (then the tile gathers); the
      // choice depends on the tile only (uniform across the workgroup, so are
      // the barriers).
      constexpr int ES = static_cast<int>(sizeof(InT));
      auto span_copy = [&]() -> const unsigned char* {
        const int base0 = t0 * a.hop - a.pad;  // first sample of the tile
        const int span = (nvalid - 1) * a.hop + NF;
        const long long xa = static_cast<long long>(reinterpret_cast<uintptr_t>(x));
        const long long lo = xa + static_cast<long long>(base0) * ES;  // may lie before x[0]
        const long long hi = lo + static_cast<long long>(span) * ES;
        const long long sig_hi = xa + static_cast<long long>(L) * ES;
        if (lo % (2 * ES) != 0 || (a.hop % 2) != 0) return nullptr;
        // whole 16-byte chunks inside the signal: rounded outwards where that
        // stays inside it, else inwards
        long long g_lo = (lo > xa ? lo : xa) & ~15LL;
        if (g_lo < xa) g_lo += 16;
        long long g_hi = ((hi < sig_hi ? hi : sig_hi) + 15) & ~15LL;
        if (g_hi > sig_hi) g_hi -= 16;
        const long long v0 = lo & ~15LL;  // the global address LDS byte 0 stands for
        const int n16 = g_hi > g_lo ? static_cast<int>((g_hi - g_lo) >> 4) : 0;
        unsigned char* dst = lds + (g_lo - v0);
        for (int c = wave; c * 64 < n16; c += NW) {
          const int q = c * 64 + lane;
          if (q < n16)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g_lo + static_cast<long long>(q) * 16),
                                             dst + c * 1024, 16, 0, 0);
        }
        // positions [0, qa) and [qb, span) of the span are filled per sample
        const int qa = n16 ? (g_lo > lo ? static_cast<int>((g_lo - lo) / ES) : 0) : span;
        const int qb = n16 ? (g_hi < hi ? static_cast<int>((g_hi - lo) / ES) : span) : span;
        const int nfill = qa + (span - qb);
        unsigned char* r0 = lds + (lo - v0);
        constexpr int KF = 4;
        for (int q0 = 0; q0 < nfill; q0 += KF * NT) {
          InT fv[KF];
#pragma unroll
          for (int k = 0; k < KF; ++k) {
            const int idx = q0 + k * NT + tid;
            const int q = idx < qa ? idx : qb + (idx - qa);
            fv[k] = idx < nfill ? padded_value(x, base0 + q, L, a.zpad, a.pad_mode) : InT(0);
          }
#pragma unroll
          for (int k = 0; k < KF; ++k) {
            const int idx = q0 + k * NT + tid;
            const int q = idx < qa ? idx : qb + (idx - qa);
            if (idx < nfill) *reinterpret_cast<InT*>(r0 + q * ES) = fv[k];
          }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the copies and fills have landed
        __syncthreads();
        return r0;
      };
      if constexpr (kHoist) {
        // Every frame of this thread is loaded before any is computed.
        constexpr int RMAX = (64 + SLOTS - 1) / SLOTS;
        float2 sb[RMAX][N1];
        const unsigned char* r0 = COPY ? span_copy() : nullptr;
        if (r0) {
          if (p1) {
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
              const int f = slot + SLOTS * r;
              if (f < nvalid) {
#pragma unroll
                for (int n1 = 0; n1 < N1; ++n1)
                  sb[r][n1] = lds_pair_raw<InT>(r0 + (f * a.hop + 2 * (N2 * n1 + n2)) * ES);
              }
            }
          }
          __syncthreads();  // the copy is consumed: Y may overwrite it
        } else if (p1) {
#pragma unroll
          for (int r = 0; r < RMAX; ++r)
            if (slot + SLOTS * r < nvalid) fetch(slot + SLOTS * r, sb[r]);
        }
        if (p1) {
#pragma unroll
          for (int r = 0; r < RMAX; ++r)
            if (slot + SLOTS * r < nvalid) compute(slot + SLOTS * r, sb[r]);
        }
      } else {
        // the tables land in LDS while the samples load
        if constexpr (kTabLds) {
          for (int c = wave; c < M / 64; c += NW)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const float*>(a.win2) + c * 256 + lane * 4,
                                             lds + a.tab_lds + c * 1024, 16, 0, 0);
        }
        // COPY: tiles of at most one frame per pass-1 thread copy their span
        const unsigned char* r0 = (COPY && nvalid <= SLOTS) ? span_copy() : nullptr;
        if (r0) {
          float2 s0[N1];
          if (p1 && slot < nvalid) {
#pragma unroll
            for (int n1 = 0; n1 < N1; ++n1) s0[n1] = lds_pair_raw<InT>(r0 + (slot * a.hop + 2 * (N2 * n1 + n2)) * ES);
          }
          __syncthreads();  // the copy is consumed: Y may overwrite it
          if (p1 && slot < nvalid) compute(slot, s0);
        } else if constexpr (kTabLds) {
          float2 s0[N1];
          if (p1 && slot < nvalid) fetch(slot, s0);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
          if (p1) {
            for (int f = slot; f < nvalid; f += SLOTS) {
              if (f != slot) fetch(f, s0);
              compute(f, s0);
            }
          }
        } else if (p1) {
          for (int f = slot; f < nvalid; f += SLOTS) {
            float2 s0[N1];
            fetch(f, s0);
            compute(f, s0);
          }
        }
      }
    }
    __syncthreads();

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(2);  // second-pass DFTs
    // ---- pass 2: N2-point DFTs, real split, power -> P (aliases Y) --
    const bool has = f2 < nvalid;
    if constexpr (ROWS) {
      // Row layout: thread (f2, k1 = p) transforms row k1 alone.  The split
      // of bin k = k1 + N1*j needs Z[M - k], which lies in row N1 - k1 at
      // index N2-1-j (row 0: itself, index (N2-j) mod N2; row N1/2: itself,
      // index N2-1-j).  A frame's N1 threads are N1 consecutive lanes of one
      // wave, so the mirrored values come from the partner lane
      // (ds_bpermute).  Rows k1 and N1-k1 share their N2 bin pairs: k1 <
      // N1/2 takes ceil(N2/2) of them, N1-k1 the other floor(N2/2); row
      // N1/2 has ceil(N2/2) pairs, row 0 floor(N2/2) + 1 (bin 0 with bin M).
      constexpr int CH = (N2 + 1) / 2;
      constexpr int CF = N2 / 2;
      constexpr int CP = CF + 1;  // most pairs of any thread (row 0)
      const int k1 = p;
      float2 za[N2], wv[kTwPrefetch ? CP : 1];
      auto tw_at = [&](int idx, int k) -> float2 {
        return kTwPrefetch ? wv[kTwPrefetch ? idx : 0] : (kTwLds ? twn_l[k] : a.tw_n[k]);
      };
      if (has) {
        if constexpr (kTwPrefetch) {  // split twiddles load under the DFT
#pragma unroll
          for (int j = 0; j < CP; ++j) wv[j] = a.tw_n[k1 + N1 * j];  // k1 + N1*j < M
        }
        const float2* ra = Y + f2 * SY + k1 * RS;
#pragma unroll
        for (int j = 0; j < N2; ++j) za[j] = ra[j];
        Dft<N2>::run(za);
      }
      // pv[j] = the partner row's Z at index N2-1-j (every lane takes part;
      // a frame's lanes all have the same `has`)
      const int partner = ((lane & ~(N1 - 1)) | ((N1 - k1) & (N1 - 1))) * 4;
      float2 pv[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j)
        pv[j] = make_float2(
            __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(za[N2 - 1 - j].x))),
            __int_as_float(__builtin_amdgcn_ds_bpermute(partner, __float_as_int(za[N2 - 1 - j].y))));
      if constexpr (kTwLds) __builtin_amdgcn_s_waitcnt(0);  // the twiddle copies have landed
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);  // split
      __syncthreads();
      // every read of the exchange buffer is done: weights into LDS behind
      // the power tile while the split runs, and the mel stage's overrun
      for (int c = wave; c < a.w_chunks; c += NW)
        __builtin_amdgcn_global_load_lds(a.blk_w + c * 256 + lane * 4, P + a.w_lds + c * 256, 16, 0, 0);
      if (tid < kMelTileOverrun) P[nvalid * SP + tid] = 0.0f;
      static_assert(SP == K, "power rows without a pad to clear");
      if (has) {
        float* prow = P + f2 * SP;
        const float hp = a.half_power;
        const int lim = k1 == 0 ? CP : (k1 <= N1 / 2 ? CH : CF);
#pragma unroll
        for (int j = 0; j < CP; ++j) {
          if (j < lim) {
            const float2 zm = k1 == 0 ? (j == 0 ? za[0] : pv[j - 1]) : pv[j < CH ? j : CH - 1];
            const int k = k1 + N1 * j;
            split_pair<PMODE>(prow + k, prow + (M - k), za[j], zm, tw_at(j, k), hp);
          }
        }
      }
    } else {
      // Unified split schedule: lanes with p != 0 pair bins p + N1*k2 (row p)
      // with M - that (row N1 - p); lanes with p == 0 own the self-paired rows 0
      // and N1/2 and walk the same N2 iterations with their rows permuted
      // (k2 < CA: row 0's pairs, k2 >= CA: row N1/2's), plus one extra pair.
      // One instruction stream for every lane: no divergent branches.
      constexpr int CA = N2 / 2 + 1;        // row 0 pairs of the p == 0 lanes
      constexpr int D2 = N1 / 2 - N1 * CA;  // bin offset of row N1/2's pairs there
      constexpr int JX = N2 - CA;           // index of row N1/2's extra pair
      const bool p0 = (p == 0);
      const int off_lo = p;                 // bin = off + N1*k2 for k2 < CA
      const int off_hi = p0 ? D2 : p;       // ... and for k2 >= CA
      float2 za[N2], zb[N2], wv[kTwPrefetch ? N2 + 1 : 1];
      auto tw_at = [&](int idx, int k) -> float2 {
        return kTwPrefetch ? wv[kTwPrefetch ? idx : 0] : (kTwLds ? twn_l[k] : a.tw_n[k]);
      };
      if (has) {
        if constexpr (kTwPrefetch) {  // split twiddles load under the DFTs
#pragma unroll
          for (int k2 = 0; k2 < N2; ++k2) wv[k2] = a.tw_n[(k2 < CA ? off_lo : off_hi) + N1 * k2];
          wv[N2] = a.tw_n[N1 / 2 + N1 * JX];
        }
        const int ka = p;
        const int kb = (p == 0) ? N1 / 2 : N1 - p;
        const float2* ra = Y + f2 * SY + ka * RS;
        const float2* rb = Y + f2 * SY + kb * RS;
#pragma unroll
        for (int j = 0; j < N2; ++j) {
          za[j] = ra[j];
          zb[j] = rb[j];
        }
        Dft<N2>::run(za);
        Dft<N2>::run(zb);
      }
      // (the twiddle copies have landed: a wave without samples to load in
      // pass 1 has not waited for its loads yet)
      if constexpr (kTwLds) __builtin_amdgcn_s_waitcnt(0);
      if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);  // split
      __syncthreads();
      // Every read of the exchange buffer is done: stream the mel weights into
      // LDS behind the power tile (direct global -> LDS loads, 1 KB per wave
      // instruction, lane l's 16 bytes at l*16), landing while the split runs.
      for (int c = wave; c < a.w_chunks; c += NW)
        __builtin_amdgcn_global_load_lds(a.blk_w + c * 256 + lane * 4, P + a.w_lds + c * 256, 16, 0, 0);
      // the mel stage may read up to kMelTileOverrun - 1 floats past the last
      // valid frame's row: keep them 0 (in a ragged last tile that is the
      // unwritten row nvalid, else the slack after the tile)
      if (tid < kMelTileOverrun) P[nvalid * SP + tid] = 0.0f;
      if (has) {
        float* prow = P + f2 * SP;
        if constexpr (SP > K) {
          if (p == 0) {
#pragma unroll
            for (int j = K; j < SP; ++j) prow[j] = 0.0f;  // row pad
          }
        }
        const float hp = a.half_power;
        // bin k = off + N1*k2 and its mirror M - k, as per-lane bases plus
        // compile-time (non-negative) offsets
        float* pk_lo = prow + off_lo;
        float* pk_hi = prow + off_hi;
        float* pm_lo = prow + (M - off_lo - N1 * (N2 - 1));
        float* pm_hi = prow + (M - off_hi - N1 * (N2 - 1));
#pragma unroll
        for (int k2 = 0; k2 < N2; ++k2) {
          float2 zk, zm;
          if (k2 < CA) {
            zk = za[k2];
            zm = p0 ? za[(N2 - k2) % N2] : zb[N2 - 1 - k2];
          } else {
            zk = p0 ? zb[k2 - CA] : za[k2];
            zm = p0 ? zb[N2 - 1 - (k2 - CA)] : zb[N2 - 1 - k2];
          }
          const int k = (k2 < CA ? off_lo : off_hi) + N1 * k2;
          float* pk = (k2 < CA ? pk_lo : pk_hi) + N1 * k2;
          float* pm = (k2 < CA ? pm_lo : pm_hi) + N1 * (N2 - 1 - k2);
          split_pair<PMODE>(pk, pm, zk, zm, tw_at(k2, k), hp);
        }
        if (p0) {
          constexpr int k = N1 / 2 + N1 * JX;
          split_pair<PMODE>(prow + k, prow + (M - k), zb[JX], zb[N2 - 1 - JX], tw_at(N2, k), hp);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the weight copies have landed in LDS
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);  // mel stage
    __syncthreads();

    // ---- mel projection on the matrix cores: each wave its filter blocks,
    //      16-frame column groups across the tile ---------------------------
    {
      CInt* tbl = (CInt*)(a.mel_tbl);  // address-space cast: scalar loads
      // The plan shares the blocks out over kMelWaves waves.  The row layout
      // spreads them over its 8 waves (waves w and w + 4 take alternate
      // blocks of wave w's share) once the tile has two or more column
      // groups, or there are blocks for every wave (8 x 480000 at n_fft 400:
      // 16.2 against 16.7 us; 1 x 480000: 7.9 against 8.2 us; n_fft 2048,
      // 64 x 220500: 89.9 against 90.8 us; with 5 blocks and 1-column tiles
      // the same or slower).
      const int nfb = (G + 15) >> 4;
      const long long obase = static_cast<long long>(b) * a.n_mels * a.n_frames + t0;  // element offset
      if (a.mel_valu) {
        // the vector units, wave w taking its 8/NW shares of the filter
        // quads (a tile's frames, at most 64, fit one wave's lanes)
        static_assert(kMelShares % NW == 0, "whole shares per wave");
        CInt* qt = (CInt*)(a.quad_tbl);
        CFloat* qw = (CFloat*)(a.quad_w);
        const int qb = qt[wave * (kMelShares / NW)], qe = qt[(wave + 1) * (kMelShares / NW)];
        if (a.out_f16)
          mel_valu<SP, _Float16>(P, qt, qw, nvalid, lane, static_cast<_Float16*>(a.out) + obase, a.n_frames,
                                 a.n_mels, qb, qe);
        else
          mel_valu<SP, float>(P, qt, qw, nvalid, lane, static_cast<float*>(a.out) + obase, a.n_frames,
                              a.n_mels, qb, qe);
        return;
      }
      const bool mel8 = ROWS && (nfb >= 2 || tbl[kMelWaves] >= 2 * kMelWaves);
      const int mw = mel8 ? (wave & 3) : wave;
      const int bb = mw < kMelWaves ? tbl[mw] + (mel8 ? (wave >> 2) : 0) : 0;
      const int be = mw < kMelWaves ? tbl[mw + 1] : 0;
      const int bstep = mel8 ? 2 : 1;
      CInt* blk = tbl + 8;
      constexpr bool GW = M >= kMelGlobalWeightsFrom;
      const float* WL = GW ? a.blk_w : P + a.w_lds;
      // this wave's staging area (mel_stage_floats)
      float* stg = P + a.w_lds + a.w_chunks * 256 + wave * (ROWS ? 16 * (16 * nfb + 1) : kMelStageFloats);
      static_assert(kMelStageMinFrames == 33, "staging is chosen for 3 and 4 column groups");
      switch (nfb) {
#define FM_MEL_CALL(NFB, STAGE)                                                                \
  if (a.out_f16)                                                                              \
    mel_blocks<SP, NFB, STAGE, GW, _Float16>(P, WL, stg, G, nvalid, lane,                      \
                                         static_cast<_Float16*>(a.out) + obase, a.n_frames,   \
                                         a.n_mels, blk, bb, be, bstep);                       \
  else                                                                                        \
    mel_blocks<SP, NFB, STAGE, GW, float>(P, WL, stg, G, nvalid, lane,                        \
                                      static_cast<float*>(a.out) + obase, a.n_frames, a.n_mels, \
                                      blk, bb, be, bstep)
        case 1: FM_MEL_CALL(1, false); break;
        case 2: FM_MEL_CALL(2, false); break;
        case 3: FM_MEL_CALL(3, true); break;
        default: FM_MEL_CALL(4, true); break;
#undef FM_MEL_CALL
      }
    }
  }
}

}  // namespace

// Kernel entry of one FFT shape for an input type, a power mode (0: p = 2,
// 1: p = 1, 2: general p), the tile-copy variant (only for shapes that
// support it) and the second pass's layout (rows: one thread per row, 512
// threads; else one per pair of rows); instantiated in fm_shape_<N1>x<N2>.hip.
template <int N1, int N2>
void* kernel_for(int in_dtype, int pmode, bool copy, bool rows, bool prio) {
  // (the phase-priority variant is built for the tile-copy kernels only)
  auto pick = [prio](auto in_tag, auto copy_tag, auto rows_tag, int pm) -> void* {
    using InT = decltype(in_tag);
    constexpr bool C = decltype(copy_tag)::value;
    constexpr bool R = decltype(rows_tag)::value;
    if constexpr (C) {
      if (prio) {
        if (pm == 0) return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 0, C, R, true>);
        if (pm == 1) return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 1, C, R, true>);
        return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 2, C, R, true>);
      }
    }
    if (pm == 0) return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 0, C, R, false>);
    if (pm == 1) return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 1, C, R, false>);
    return reinterpret_cast<void*>(&mel_forward_kernel<N1, N2, InT, 2, C, R, false>);
  };
  auto by_layout = [&](auto in_tag, auto copy_tag) -> void* {
    if constexpr (kRowsCapable<N1, N2>) {
      if (rows) return pick(in_tag, copy_tag, std::true_type{}, pmode);
    } else {
      if (rows) return nullptr;
    }
    return pick(in_tag, copy_tag, std::false_type{}, pmode);
  };
  using Yes = std::integral_constant<bool, kCopyCapable<N1, N2>>;
  using No = std::false_type;
  if (copy && kCopyCapable<N1, N2>) {
    if (in_dtype == FM_I16) return by_layout(int16_t{}, Yes{});
    return by_layout(float{}, Yes{});
  }
  if (in_dtype == FM_I16) return by_layout(int16_t{}, No{});
  return by_layout(float{}, No{});
}

// Shapes built into the library (n_fft/2 = N1 * N2).
#define FM_FOR_EACH_SHAPE(X) \
  X(8, 4) X(8, 8) X(8, 16) X(8, 25) X(16, 16) X(32, 16) X(32, 32) X(64, 32)
#define FM_DECLARE_SHAPE(A, B) extern template void* kernel_for<A, B>(int, int, bool, bool, bool);
FM_FOR_EACH_SHAPE(FM_DECLARE_SHAPE)
#undef FM_DECLARE_SHAPE

}  // namespace fm
