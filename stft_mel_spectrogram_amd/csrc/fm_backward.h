// Backward of the fused mel-spectrogram for gfx950 (MI355X): the gradient
// of sum(grad_out * mel(x)) with respect to the float32 signal x.
//
// The forward chain (padding, framing, window w, one-sided DFT X, |X|^p,
// mel projection with filterbank W) is linear up to |X|^p, so the gradient
// is its adjoint applied step by step, in reverse:
//   dP_t[k] = sum_m W[m,k] g[m,t]          (each bin lies in <= 2 filters)
//   G_t[k]  = p |X_t[k]|^(p-2) X_t[k] dP_t[k]   (complex: dRe + i dIm)
//   d_t[n]  = Re sum_{k<=N/2} G_t[k] exp(+2 pi i n k / N)
//   dx_pad[t*hop + n] += w[n] d_t[n],  dx = adjoint of the padding map.
// X is recomputed from x (the forward's register FFT: pass 1, pass 2 and
// the real-spectrum split).  d is the inverse real FFT of a Hermitian
// spectrum, carried by a complex inverse FFT of M = N/2 points on
// z[m] = d[2m] + i d[2m+1], with the inverse of the split,
//   C[k]   = E + i V,  C[M-k] = conj(E - i V),
//   E = H[k] + conj H[M-k],  V = exp(+2 pi i k/N) (H[k] - conj H[M-k]),
// H[k] = G[k]/2 (0 < k < M), H[0] = Re G[0], H[M] = Re G[M]; then the two
// register passes run backwards (n2-point inverse DFTs of each row k1,
// exchange, twiddle exp(+2 pi i n2 k1 / M), n1-point inverse DFTs).  Each
// thread overwrites exactly the exchange-buffer slots it read, so the
// windowed frame gradients w[n] d_t[n] replace the spectrum in place.
//
// Overlap-add is a gather: every output sample sums the (at most
// ceil(n_fft/hop)) frames that cover it, in a fixed order, so the result is
// deterministic and needs no atomics or zero-fill.
//   * main workgroups each own a run of samples (their tile of frames' hops)
//     and recompute the frames that reach into it: the tile plus the
//     floor((n_fft-1)/hop) frames before it, in one pass, or, when more
//     frames overlap than a pass holds (small hops), in several passes that
//     accumulate the owned samples in LDS;
//   * one edge workgroup per signal owns the first and last n_fft/2 + 1
//     samples, where the centre padding folds gradients of padded positions
//     back onto signal samples (reflect: the mirrored sample; circular: the
//     wrapped one; replicate: the end samples collect every padded position
//     on their side, summed by a block reduction).  It runs the frames that
//     reach its zones in passes of up to one chunk and accumulates per
//     sample in LDS.
#pragma once

#include "fm_kernel.h"

namespace fm {

struct BArgs {
  const float* in;       // [B, L] signal
  const float* gout;     // [B, n_mels, T] gradient of the output
  float* gin;            // [B, L] gradient of the signal (every sample written)
  const float2* win2;    // [M] 0.5*(w[2m], w[2m+1])
  const float2* tw_m;    // [M] exp(-2 pi i j / M)
  const float2* tw_n;    // [M] exp(-2 pi i k / N)
  const BinTap* taps;    // [M + 1]
  long long length;
  int n_frames;
  int hop;
  int pad;               // first frame's offset before sample 0
  int zpad;              // zero samples added on both sides
  int pad_mode;
  int n_mels;
  int tile;              // frames whose hops a main workgroup owns
  int halo;              // frames before the tile that reach into it
  int tiles_per_signal;
  int n_edge;            // edge workgroups (first in the grid), one per signal
  int edge;              // samples at each end owned by the edge workgroups
  int edge_split;        // 1: two edge workgroups per signal (head, tail)
  int whole;             // 1: the edge workgroup owns the whole signal
  int chunk;             // frames per pass
  int vec_ok;            // interior frames may use paired loads
  int g_off;             // LDS float offset of the bin-gradient tile dP[f][k]
  int gt_off;            // LDS float offset of the output-gradient tile g[m][f]
  int acc_off;           // LDS float offset of the edge accumulators
  int multi;             // 1: a main workgroup's frames take several passes; its
                         // samples accumulate in LDS at oacc_off
  int oacc_off;
  float power;
  float half_power;
};

namespace {

// Scale s with G = s * X for the gradient of |X|^p (PMODE as in the
// forward): p = 2: 2 dP; p = 1: dP / |X|; general p: p dP |X|^(p-2).  Where
// X = 0 and p != 2 the gradient is 0.
template <int PMODE>
__device__ __forceinline__ float grad_scale(float2 x, float dP, float power, float hp) {
  if constexpr (PMODE == 0) {
    return 2.0f * dP;
  } else {
    const float sq = fmaf(x.x, x.x, x.y * x.y);
    if constexpr (PMODE == 1) {
      return sq > 0.0f ? dP * __builtin_amdgcn_rsqf(sq) : 0.0f;  // v_rsq_f32, 1 ulp
    } else {
      // |X|^(p-2) = 2^((p/2 - 1) log2 |X|^2)
      return sq > 0.0f ? power * dP * __builtin_amdgcn_exp2f((hp - 1.0f) * __builtin_amdgcn_logf(sq))
                       : 0.0f;
    }
  }
}

// Pairs of the gradient split scheduled together (see the loop).
constexpr int kBwdPairGroup = 4;

template <int N1, int N2, int PMODE>
__global__ __launch_bounds__(kBwdThreads, bwd_min_waves(N1, N2)) void mel_backward_kernel(BArgs a) {
  constexpr int M = N1 * N2;
  constexpr int K = M + 1;        // one-sided bins; odd: the dP tile's frame stride
  constexpr int SY = bwd_exchange_stride(M);
  constexpr int DS = 2 * SY;      // float stride of a frame of frame gradients
  constexpr int NF = 2 * M;       // n_fft
  constexpr int NPAIR = N1 / 2;
  constexpr int NT = kBwdThreads;
  constexpr int NW = NT / 64;
  constexpr int SLOTS = NT / N2;
  constexpr bool kHoist = N1 <= 8;
  constexpr int CAP = bwd_chunk_cap(N1, N2, NT);
  constexpr bool kRowPass2 = N1 <= 8;  // pass 2: a thread per row (else per row pair)
  constexpr int CA = N2 / 2 + 1;
  constexpr int D2 = N1 / 2 - N1 * CA;
  constexpr int JX = N2 - CA;

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float2* Y = reinterpret_cast<float2*>(lds);
  float* D = reinterpret_cast<float*>(lds);  // D[f][n], aliases Y
  float* dPt = reinterpret_cast<float*>(lds) + a.g_off;  // dP[f][k]
  float* Gt = reinterpret_cast<float*>(lds) + a.gt_off;  // g[m][f] of the pass
  float* acc = reinterpret_cast<float*>(lds) + a.acc_off;
  float* red = acc + 2 * a.edge;

  const int tid = threadIdx.x;
  const int L = static_cast<int>(a.length);
  const int T = a.n_frames;
  const int hop = a.hop;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- this workgroup's signal, frame segments and owned samples ----------
  // logical workgroup id in the XCD-aware order (edge workgroups first)
  const int wid = __builtin_amdgcn_readfirstlane(xcd_tile_order(blockIdx.x, gridDim.x));
  const bool edge_wg = wid < a.n_edge;
  int b, seg0_lo, seg0_hi, seg1_lo = 0, seg1_hi = 0, own_lo = 0, own_hi = 0;
  int n_acc = 0, s_lo = 0, s_hi = 0;  // edge: accumulator slots, owned ones
  if (edge_wg) {
    // side 0: the head zone [0, edge), side 1: the tail zone [L - edge, L),
    // each in a workgroup of its own (edge_split), else both in one
    const int side = a.edge_split ? (wid & 1) : -1;
    b = a.edge_split ? (wid >> 1) : wid;
    n_acc = a.whole ? L : 2 * a.edge;
    s_lo = side == 1 ? a.edge : 0;
    s_hi = side == 0 ? a.edge : n_acc;
    // frames reaching the head zone and the tail zone
    const int th = min(T, (a.edge + a.pad + hop - 1) / hop);
    const int num = L - a.edge + a.pad - NF;
    const int tt = num < 0 ? 0 : num / hop + 1;
    if (side == 0) {
      seg0_lo = 0;
      seg0_hi = th;
    } else if (side == 1) {
      seg0_lo = tt;
      seg0_hi = T;
    } else if (a.whole || th >= tt) {
      seg0_lo = 0;
      seg0_hi = T;
    } else {
      seg0_lo = 0;
      seg0_hi = th;
      seg1_lo = tt;
      seg1_hi = T;
    }
    for (int s = s_lo + tid; s < s_hi; s += NT) acc[s] = 0.0f;
  } else {
    const int w = wid - a.n_edge;
    // (the division expands to vector code: bring the uniform result back to
    // a scalar register)
    b = __builtin_amdgcn_readfirstlane(w / a.tiles_per_signal);
    const int ti = w - b * a.tiles_per_signal;
    const int t0 = ti * a.tile;
    seg0_lo = max(0, t0 - a.halo);
    seg0_hi = min(T, t0 + a.tile);
    own_lo = ti == 0 ? 0 : t0 * hop - a.pad;
    own_hi = ti == a.tiles_per_signal - 1 ? L : (t0 + a.tile) * hop - a.pad;
    own_lo = max(own_lo, a.edge);
    own_hi = min(own_hi, L - a.edge);
  }
  const float* x = a.in + static_cast<long long>(b) * L;
  const float* g = a.gout + static_cast<long long>(b) * a.n_mels * T;
  float* gx = a.gin + static_cast<long long>(b) * L;

  // Sum of the frame gradients of frames [ca, ca + nf) at padded position q
  // (q = thi*hop + qr, 0 <= qr < hop), latest frame first: at most
  // ceil(n_fft / hop) frames, as a fixed predicated loop so that the reads
  // are in flight together.
  const int nover = (NF + hop - 1) / hop;
  const int dstep = hop - DS;  // index step to the previous frame's sample
  auto gather_at = [&](int ca, int nf, int thi, int qr) -> float {
    const int t = min(thi, ca + nf - 1);
    const int n = qr + (thi - t) * hop;
    const int idx = (t - ca) * DS + n;
    // four frames' reads issued together, then summed in order
    float v[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ok[j] = t - j >= ca && n + j * hop < NF;
      v[j] = D[ok[j] ? idx + j * dstep : 0];
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += ok[j] ? v[j] : 0.0f;
    const int jmax = min(nover, t - ca + 1);  // (hop < n_fft / 4)
    for (int j = 4; j < jmax; ++j)
      if (n + j * hop < NF) s += D[idx + j * dstep];
    return s;
  };
  auto gather = [&](int ca, int nf, int i) -> float {  // i: sample position
    const int q = i + a.pad;
    if (q < 0) return 0.0f;
    const int thi = q / hop;
    return gather_at(ca, nf, thi, q - thi * hop);
  };

  // Every phase derives its lane indices from its own copy of the thread
  // index, which the compiler cannot prove invariant: addresses and table
  // loads stay inside their phase instead of being hoisted out of it (and out
  // of the pass loop) and held in registers, or spilled, meanwhile.
  auto opaque_tid = [&]() {
    int v = tid;
    asm volatile("" : "+v"(v));
    return v;
  };

  // Pass 2 with one thread per (frame, row k1) (shapes with N1 <= 8): the
  // row's N2-point DFT, then the split with the mirrored bins M - k read from
  // the partner row (row N1 - k1, or the row itself for k1 = 0 and N1/2)
  // through LDS, the gradient of |X|^p and the inverse-split values C[k] and
  // C[M - k], each pair computed by one of the two threads, and the row's
  // inverse DFT.  Partners are lanes of the same wave, and a wave's LDS
  // operations complete in order, so no barrier is needed inside.
  auto pass2_rows = [&](int nf) {
    const int t2 = opaque_tid();
    const int f2 = t2 / N1;
    const int r = t2 - f2 * N1;
    if (f2 >= nf) return;
    const int rp = (N1 - r) & (N1 - 1);  // partner row
    float2* row = Y + f2 * SY + r * N2;
    const float2* prow = Y + f2 * SY + rp * N2;
    float2 z[N2];
#pragma unroll
    for (int j = 0; j < N2; ++j) z[j] = row[j];
    Dft<N2>::run(z);
#pragma unroll
    for (int j = 0; j < N2; ++j) row[j] = z[j];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's rows are written
    __builtin_amdgcn_wave_barrier();
    // Each pair (k, M - k) is computed once: this thread takes its bins
    // k2 < hmine and sends C[M - k] to the mirrored slot (in the partner row,
    // or its own row for the self-paired rows 0 and N1/2); the partner's pairs
    // fill the rest of this row.
    const bool r0 = (r == 0);
    const int hmine = r0 ? N2 / 2 + 1 : (r <= N1 / 2 ? (N2 + 1) / 2 : N2 / 2);
    constexpr int HMAX = N2 / 2 + 1;
    // zp[k2] = the mirror of bin r + N1*k2: row 0 -> its index (N2 - k2) % N2
    // (k2 = 0: bin M, i.e. Z[0]); other rows -> index N2 - 1 - k2 of the
    // partner row (the choice is made on the LDS address, not on registers)
    float2 zp[HMAX];
    float2* mdst[HMAX];
#pragma unroll
    for (int j = 0; j < HMAX; ++j) {
      mdst[j] = const_cast<float2*>(prow) + (r0 ? (N2 - j) % N2 : N2 - 1 - j);
      zp[j] = *mdst[j];
    }
    // split twiddle exp(-2 pi i k/N), k = r + N1*k2: the table value of r times
    // the compile-time rotation exp(-2 pi i k2/(2 N2))
    const float2 w_r = a.tw_n[r];
    const float* dprow = dPt + f2 * K;
    const float* dk = dprow + r;        // dP[k]     = dk[N1*k2]
    const float* dm = dprow + (M - r);  // dP[M - k] = dm[-N1*k2]
    static_for<0, HMAX>([&](auto k2c) {
      constexpr int k2 = decltype(k2c)::value;
      const float2 zk = z[k2];
      const float2 zm = zp[k2];
      const float2 w = twiddle<k2, 2 * N2>(w_r);
      const bool dc = r0 && k2 == 0;
      const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);   // Z[k] + conj Z[M-k]
      const float2 o = make_float2(zk.x - zm.x, zk.y + zm.y);   // Z[k] - conj Z[M-k]
      const float2 v = cmul(w, o);
      const float2 xk = make_float2(e.x + v.y, e.y - v.x);      // X[k]   = e - i v
      const float2 xm = make_float2(e.x - v.y, -(e.y + v.x));   // X[M-k] = conj(e + i v)
      const float sk = grad_scale<PMODE>(xk, dk[N1 * k2], a.power, a.half_power);
      const float sm = grad_scale<PMODE>(xm, dm[-N1 * k2], a.power, a.half_power);
      const float hs = dc ? 1.0f : 0.5f;
      const float2 hk = make_float2(hs * sk * xk.x, dc ? 0.0f : hs * sk * xk.y);
      const float2 hm = make_float2(hs * sm * xm.x, dc ? 0.0f : hs * sm * xm.y);
      const float2 E = make_float2(hk.x + hm.x, hk.y - hm.y);   // H[k] + conj H[M-k]
      const float2 O = make_float2(hk.x - hm.x, hk.y + hm.y);   // H[k] - conj H[M-k]
      const float2 V = cmul(make_float2(w.x, -w.y), O);         // exp(+2 pi i k/N) O
      if (k2 < hmine) {
        z[k2] = make_float2(E.x - V.y, E.y + V.x);              // C[k]   = E + i V
        *mdst[k2] = make_float2(E.x + V.y, V.x - E.y);          // C[M-k] = conj(E - i V)
      }
      if constexpr (k2 % kBwdPairGroup == kBwdPairGroup - 1) __builtin_amdgcn_sched_barrier(0);
    });
    // the rest of this row: the values the partner (or this thread, as
    // mirrors) wrote; every read of Z from LDS in this wave came first
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < N2; ++j) {
      const float2 t = row[j];
      z[j] = j < hmine ? z[j] : t;
    }
    // inverse N2-point DFT over k2 (conjugate, forward DFT, conjugate); the
    // partner's reads of this row were issued before these writes
#pragma unroll
    for (int j = 0; j < N2; ++j) z[j].y = -z[j].y;
    Dft<N2>::run(z);
#pragma unroll
    for (int j = 0; j < N2; ++j) row[j] = make_float2(z[j].x, -z[j].y);
  };

  int cur = seg0_lo, seg_hi = seg0_hi;
  bool second = false;
  for (;;) {
    if (cur >= seg_hi) {
      if (!second && seg1_hi > seg1_lo) {
        second = true;
        cur = seg1_lo;
        seg_hi = seg1_hi;
      } else {
        break;
      }
    }
    const int ca = cur;
    const int nf = min(a.chunk, seg_hi - cur);
    cur += nf;
    const int lane = opaque_tid() & 63;

    // ---- pass 1 (forward transform): window, N1-point DFTs, twiddle -> Y --
    {
      const int t1 = opaque_tid();
      const int n2v = t1 % N2;  // fixed n2; frames slot, slot + SLOTS, ...
      const int slot = t1 / N2;
      const bool p1 = slot < SLOTS;
      float2 win[kHoist ? N1 : 1], twv[kHoist ? N1 : 1];
      if constexpr (kHoist) {
#pragma unroll
        for (int n1 = 0; n1 < N1; ++n1) win[n1] = a.win2[N2 * n1 + n2v];
        twv[0] = make_float2(1.0f, 0.0f);
#pragma unroll
        for (int k1 = 1; k1 < N1; ++k1) twv[k1] = a.tw_m[n2v * k1];
      }
      auto fetch = [&](int f, float2 (&s)[N1]) {
        const int base = (ca + f) * hop - a.pad;
        if (a.vec_ok && base >= 0 && base + NF <= L) {
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1) s[n1] = load_pair(x, base + 2 * (N2 * n1 + n2v));
        } else {
#pragma unroll
          for (int n1 = 0; n1 < N1; ++n1) {
            const int i = base + 2 * (N2 * n1 + n2v);
            s[n1] = make_float2(padded_sample_raw(x, i, L, a.zpad, a.pad_mode),
                                padded_sample_raw(x, i + 1, L, a.zpad, a.pad_mode));
          }
        }
      };
      auto compute = [&](int f, const float2 (&s)[N1]) {
        float2 v[N1];
#pragma unroll
        for (int n1 = 0; n1 < N1; ++n1) {
          const float2 w = kHoist ? win[kHoist ? n1 : 0] : a.win2[N2 * n1 + n2v];
          v[n1] = make_float2(s[n1].x * w.x, s[n1].y * w.y);
        }
        // (large N1: keep the twiddle loads after the DFT, not above it)
        if constexpr (!kHoist) __builtin_amdgcn_sched_barrier(0);
        Dft<N1>::run(v);
        if constexpr (!kHoist) __builtin_amdgcn_sched_barrier(0);
        float2* yrow = Y + f * SY + n2v;
        yrow[0] = v[0];
#pragma unroll
        for (int k1 = 1; k1 < N1; ++k1)
          yrow[k1 * N2] = cmul(v[k1], kHoist ? twv[kHoist ? k1 : 0] : a.tw_m[n2v * k1]);
      };
      // The output-gradient tile g[m][ca .. ca+nf) goes to LDS by direct
      // global -> LDS loads (one row per wave instruction, no registers),
      // issued before the samples so that both arrive in one round trip;
      // the bin gradients are formed from it after pass 1.
      if (lane < nf) {
        for (int m = wave; m < a.n_mels; m += NW)
          __builtin_amdgcn_global_load_lds(g + static_cast<long long>(m) * T + ca + lane, Gt + m * nf, 4, 0, 0);
        if (wave == NW - 1) Gt[a.n_mels * nf + lane] = 0.0f;  // row n_mels: unused taps
      }
      if constexpr (kHoist) {
        constexpr int RMAX = (CAP + SLOTS - 1) / SLOTS;
        // (every round loads, rounds past the pass repeat its last frame: a
        // conditionally defined array would stay live around the pass loop)
        float2 sb[RMAX][N1];
        if (p1) {
#pragma unroll
          for (int r = 0; r < RMAX; ++r) fetch(min(slot + SLOTS * r, nf - 1), sb[r]);
#pragma unroll
          for (int r = 0; r < RMAX; ++r)
            if (slot + SLOTS * r < nf) compute(slot + SLOTS * r, sb[r]);
        }
      } else if (p1) {
        for (int f = slot; f < nf; f += SLOTS) {
          float2 s0[N1];
          fetch(f, s0);
          compute(f, s0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gradient-tile rows have landed
    __syncthreads();

    // ---- bin gradients dP[f][k] = sum_m W[m,k] g[m][ca+f]: thread = bin
    //      (its two taps one vector load), frames in an unrolled loop of
    //      independent LDS reads -----------------------------------------
    for (int k = opaque_tid(); k < K; k += NT) {
      const BinTap tap = a.taps[k];
      const float* g0 = Gt + tap.m0 * nf;
      const float* g1 = Gt + tap.m1 * nf;
#pragma unroll 4
      for (int f = 0; f < nf; ++f) dPt[f * K + k] = fmaf(tap.w1, g1[f], tap.w0 * g0[f]);
    }
    __syncthreads();

    // ---- pass 2, split, gradient of |X|^p, inverse split, inverse pass 2 --
    if constexpr (kRowPass2) {
      pass2_rows(nf);
      __syncthreads();
    } else {
    const int t2 = opaque_tid();
    const int f2 = t2 / NPAIR;  // frame f2, pair pv of rows
    const int pv = t2 - f2 * NPAIR;
    if (f2 < nf) {
      const bool p0 = (pv == 0);
      const int off_lo = pv;                // bin = off + N1*k2 for k2 < CA
      const int off_hi = p0 ? D2 : pv;      // ... and for k2 >= CA
      const int ka = pv;
      const int kb = p0 ? N1 / 2 : N1 - pv;
      float2* ra = Y + f2 * SY + ka * N2;
      float2* rb = Y + f2 * SY + kb * N2;
      float2 za[N2], zb[N2];
#pragma unroll
      for (int j = 0; j < N2; ++j) {
        za[j] = ra[j];
        zb[j] = rb[j];
      }
      // (long rows: one DFT's temporaries at a time)
      constexpr bool kSerialRows = N2 >= 32;
      Dft<N2>::run(za);
      if constexpr (kSerialRows) __builtin_amdgcn_sched_barrier(0);
      Dft<N2>::run(zb);
      if constexpr (kSerialRows) __builtin_amdgcn_sched_barrier(0);
      // split twiddles exp(-2 pi i k/N), k = off + N1*k2: one table value per
      // row times the compile-time rotation exp(-2 pi i k2/(2 N2))
      const float2 w_lo = a.tw_n[off_lo];
      const float2 wh = a.tw_n[p0 ? -D2 : pv];
      const float2 w_hi = p0 ? make_float2(wh.x, -wh.y) : wh;
      // dP of bin k = off + N1*k2 and of its mirror M - k, as per-lane bases
      // plus compile-time offsets
      const float* dprow = dPt + f2 * K;
      const float* dk_lo = dprow + off_lo;
      const float* dk_hi = dprow + off_hi;
      const float* dm_lo = dprow + (M - off_lo - N1 * (N2 - 1));
      const float* dm_hi = dprow + (M - off_hi - N1 * (N2 - 1));
      // (zk, zm) = (Z[k], Z[M-k]) -> (C[k], C[M-k]); w = exp(-2 pi i k/N);
      // dc: the pair (0, M)
      auto grad_pair = [&](float2 zk, float2 zm, float2 w, float dpk, float dpm, bool dc,
                           float2& ck, float2& cm) {
        const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);   // Z[k] + conj Z[M-k]
        const float2 o = make_float2(zk.x - zm.x, zk.y + zm.y);   // Z[k] - conj Z[M-k]
        const float2 v = cmul(w, o);
        const float2 xk = make_float2(e.x + v.y, e.y - v.x);      // X[k]   = e - i v
        const float2 xm = make_float2(e.x - v.y, -(e.y + v.x));   // X[M-k] = conj(e + i v)
        const float sk = grad_scale<PMODE>(xk, dpk, a.power, a.half_power);
        const float sm = grad_scale<PMODE>(xm, dpm, a.power, a.half_power);
        const float hs = dc ? 1.0f : 0.5f;
        const float2 hk = make_float2(hs * sk * xk.x, dc ? 0.0f : hs * sk * xk.y);
        const float2 hm = make_float2(hs * sm * xm.x, dc ? 0.0f : hs * sm * xm.y);
        const float2 E = make_float2(hk.x + hm.x, hk.y - hm.y);   // H[k] + conj H[M-k]
        const float2 O = make_float2(hk.x - hm.x, hk.y + hm.y);   // H[k] - conj H[M-k]
        const float2 V = cmul(make_float2(w.x, -w.y), O);         // exp(+2 pi i k/N) O
        ck = make_float2(E.x - V.y, E.y + V.x);                   // E + i V
        cm = make_float2(E.x + V.y, V.x - E.y);                   // conj(E - i V)
      };
      // Same pairing schedule as the forward split: every Z element is read
      // by exactly one pair, and its C value written back to its slot.
      static_for<0, N2>([&](auto k2c) {
        constexpr int k2 = decltype(k2c)::value;
        float2 zk, zm;
        if constexpr (k2 < CA) {
          zk = za[k2];
          zm = p0 ? za[(N2 - k2) % N2] : zb[N2 - 1 - k2];
        } else {
          zk = p0 ? zb[k2 - CA] : za[k2];
          zm = p0 ? zb[N2 - 1 - (k2 - CA)] : zb[N2 - 1 - k2];
        }
        const float2 w = twiddle<k2, 2 * N2>(k2 < CA ? w_lo : w_hi);
        const float dpk = k2 < CA ? dk_lo[N1 * k2] : dk_hi[N1 * k2];
        const float dpm = k2 < CA ? dm_lo[N1 * (N2 - 1 - k2)] : dm_hi[N1 * (N2 - 1 - k2)];
        float2 ck, cm;
        grad_pair(zk, zm, w, dpk, dpm, k2 == 0 && p0, ck, cm);
        // (stores to fixed slots of selected values: a store through a
        // selected slot would push both arrays out of registers)
        if constexpr (k2 < CA) {
          za[k2] = ck;
          za[(N2 - k2) % N2] = p0 ? cm : za[(N2 - k2) % N2];
          zb[N2 - 1 - k2] = p0 ? zb[N2 - 1 - k2] : cm;
        } else {
          za[k2] = p0 ? za[k2] : ck;
          zb[N2 - 1 - k2] = p0 ? zb[N2 - 1 - k2] : cm;
          zb[k2 - CA] = p0 ? ck : zb[k2 - CA];
          zb[N2 - 1 - (k2 - CA)] = p0 ? cm : zb[N2 - 1 - (k2 - CA)];
        }
        // keep the scheduler from hoisting every pair's loads to the top
        if constexpr (k2 % kBwdPairGroup == kBwdPairGroup - 1) __builtin_amdgcn_sched_barrier(0);
      });
      if (p0) {  // row N1/2's remaining pair: k = N1/2 + N1*JX = off_hi + N1*N2
        float2 ck, cm;
        grad_pair(zb[JX], zb[N2 - 1 - JX], twiddle<N2, 2 * N2>(w_hi), dk_hi[N1 * N2],
                  dm_hi[-N1],  // bins k and M - k
                  false, ck, cm);
        zb[JX] = ck;
        zb[N2 - 1 - JX] = cm;
      }
      // inverse N2-point DFTs over k2 (conjugate, forward DFT, conjugate)
#pragma unroll
      for (int j = 0; j < N2; ++j) {
        za[j].y = -za[j].y;
        zb[j].y = -zb[j].y;
      }
      Dft<N2>::run(za);
      if constexpr (kSerialRows) __builtin_amdgcn_sched_barrier(0);
      Dft<N2>::run(zb);
#pragma unroll
      for (int j = 0; j < N2; ++j) {
        ra[j] = make_float2(za[j].x, -za[j].y);
        rb[j] = make_float2(zb[j].x, -zb[j].y);
      }
    }
    __syncthreads();
    }

    // ---- inverse pass 1: twiddle, N1-point inverse DFTs, window -> D -------
    const int t3 = opaque_tid();
    const int n2v = t3 % N2;
    const int slot = t3 / N2;
    if (slot < SLOTS) {
      for (int f = slot; f < nf; f += SLOTS) {
        float2* col = Y + f * SY + n2v;
        float2 v[N1];
        v[0] = col[0];
#pragma unroll
        for (int k1 = 1; k1 < N1; ++k1) {
          const float2 u = col[k1 * N2];
          const float2 t = a.tw_m[n2v * k1];
          v[k1] = make_float2(fmaf(u.x, t.x, u.y * t.y), fmaf(u.y, t.x, -(u.x * t.y)));  // u conj(t)
        }
#pragma unroll
        for (int k1 = 0; k1 < N1; ++k1) v[k1].y = -v[k1].y;
        // (large N1: keep the window loads after the DFT, not above it)
        if constexpr (!kHoist) __builtin_amdgcn_sched_barrier(0);
        Dft<N1>::run(v);
        if constexpr (!kHoist) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n1 = 0; n1 < N1; ++n1) {
          const float2 w = a.win2[N2 * n1 + n2v];  // w/2: the factor 2 is restored here
          col[n1 * N2] = make_float2(2.0f * w.x * v[n1].x, -2.0f * w.y * v[n1].y);
        }
      }
    }
    __syncthreads();

    // ---- overlap-add ---------------------------------------------------------
    const int t4 = opaque_tid();
    if (!edge_wg) {
      int i = own_lo + t4;
      if (i < own_hi) {
        const int q = i + a.pad;
        int thi = q / hop, qr = q - thi * hop;
        const int dq = NT / hop, rq = NT - dq * hop;
        // several passes: each thread adds this pass's frames to its own
        // samples' accumulators (the same thread every pass, no barrier)
        float* oacc = reinterpret_cast<float*>(lds) + a.oacc_off - own_lo;
        const bool first = ca == seg0_lo;
        for (; i < own_hi; i += NT) {
          const float v = gather_at(ca, nf, thi, qr);
          if (!a.multi) __builtin_nontemporal_store(v, gx + i);
          else oacc[i] = first ? v : oacc[i] + v;
          thi += dq;
          qr += rq;
          if (qr >= hop) {
            qr -= hop;
            ++thi;
          }
        }
      }
    } else {
      // each owned sample: its own position plus the padded positions that
      // the padding map sends to it (one reflection or wrap at most)
      const int ly = L + 2 * a.zpad;
      for (int s = s_lo + t4; s < s_hi; s += NT) {
        const int j = (a.whole || s < a.edge) ? s : L - 2 * a.edge + s;
        float v = gather(ca, nf, j);
        if (a.pad_mode == FM_PAD_REFLECT) {
          const int y0 = j + a.zpad;
          if (y0 >= 1) v += gather(ca, nf, -j - 2 * a.zpad);
          if (y0 <= ly - 2) v += gather(ca, nf, 2 * (ly - 1) - j - 2 * a.zpad);
        } else if (a.pad_mode == FM_PAD_CIRCULAR) {
          v += gather(ca, nf, j - ly);
          v += gather(ca, nf, j + ly);
        }
        acc[s] += v;
      }
      if (a.pad_mode == FM_PAD_REPLICATE && a.zpad == 0) {
        // every padded position before the signal repeats sample 0, every
        // one after it sample L-1: block sums in a fixed order
        float sl = 0.0f, sr = 0.0f;
        for (int e = t4; e < nf * NF; e += NT) {
          const int f = e / NF, n = e - f * NF;
          const int i = (ca + f) * hop - a.pad + n;
          const float v = D[f * DS + n];
          if (i < 0) sl += v;
          else if (i >= L) sr += v;
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          sl += __shfl_xor(sl, o);
          sr += __shfl_xor(sr, o);
        }
        if ((t4 & 63) == 0) {
          red[wave] = sl;
          red[NW + wave] = sr;
        }
        __syncthreads();
        if (t4 == 0) {
          float tl = 0.0f, tr = 0.0f;
          for (int w = 0; w < NW; ++w) {
            tl += red[w];
            tr += red[NW + w];
          }
          acc[0] += tl;
          acc[n_acc - 1] += tr;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next pass
  }

  if (!edge_wg && a.multi) {
    const float* oacc = reinterpret_cast<const float*>(lds) + a.oacc_off - own_lo;
    for (int i = own_lo + tid; i < own_hi; i += NT) __builtin_nontemporal_store(oacc[i], gx + i);
  }
  if (edge_wg) {
    for (int s = s_lo + tid; s < s_hi; s += NT) {
      const int j = (a.whole || s < a.edge) ? s : L - 2 * a.edge + s;
      gx[j] = acc[s];
    }
  }
}

}  // namespace

// Backward kernel of one FFT shape for a power mode (0: p = 2, 1: p = 1,
// 2: general p); instantiated in fm_shape_<N1>x<N2>.hip.
template <int N1, int N2>
void* backward_kernel_for(int pmode) {
  if (pmode == 0) return reinterpret_cast<void*>(&mel_backward_kernel<N1, N2, 0>);
  if (pmode == 1) return reinterpret_cast<void*>(&mel_backward_kernel<N1, N2, 1>);
  return reinterpret_cast<void*>(&mel_backward_kernel<N1, N2, 2>);
}

#define FM_DECLARE_BWD_SHAPE(A, B) extern template void* backward_kernel_for<A, B>(int);
FM_FOR_EACH_SHAPE(FM_DECLARE_BWD_SHAPE)
#undef FM_DECLARE_BWD_SHAPE

}  // namespace fm
