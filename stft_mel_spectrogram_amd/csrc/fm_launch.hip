// Host side of the fused mel-spectrogram forward pass: plan upload, tile
// choice per call and the launch (the kernels live in fm_shape_*.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "fm_backward.h"
#include "fm_large.h"
#include "fm_pair.h"

namespace fm {

namespace {

int power_mode(const Plan& p) { return p.power == 2.0 ? 0 : (p.power == 1.0 ? 1 : 2); }

void* select_backward_kernel(const Plan& p) {
  const int pm = power_mode(p);
#define FM_SELECT_SHAPE(A, B) \
  if (p.fft.n1 == A && p.fft.n2 == B) return backward_kernel_for<A, B>(pm);
  FM_FOR_EACH_SHAPE(FM_SELECT_SHAPE)
#undef FM_SELECT_SHAPE
  return nullptr;
}

void* select_kernel(const Plan& p, int in_dtype, bool copy, bool rows, bool prio = false) {
  const int pm = power_mode(p);
#define FM_SELECT_SHAPE(A, B) \
  if (p.fft.n1 == A && p.fft.n2 == B) return kernel_for<A, B>(in_dtype, pm, copy, rows, prio);
  FM_FOR_EACH_SHAPE(FM_SELECT_SHAPE)
#undef FM_SELECT_SHAPE
  return nullptr;
}

void* select_large_kernel(const Plan& p, int in_dtype) {
  const int pm = power_mode(p);
#define FM_SELECT_LARGE(A, C, D) \
  if (p.lfft.n1 == A && p.lfft.n2 == C && p.lfft.n3 == D) \
    return large_kernel_for<A, C, D>(in_dtype, pm, p.n_mels > p.large_threads);
  FM_FOR_EACH_LARGE_SHAPE(FM_SELECT_LARGE)
#undef FM_SELECT_LARGE
  return nullptr;
}
void* select_pair_kernel(const Plan& p, int in_dtype) {
  if (p.pair_r == 20) return pair_kernel_for<20>(in_dtype, power_mode(p));
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
  e = hipDeviceGetAttribute(&p.n_cu, hipDeviceAttributeMultiprocessorCount, p.device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  const int M = p.n_fft / 2;
  // one block: win2 | tw_m | tw_n | rows | mel_w | mel blocks | block weights,
  // each 256-byte aligned
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const size_t o_win = 0;
  const size_t o_twp = o_win + al(M * sizeof(float2));
  const size_t o_twm = o_twp + al(M * sizeof(float2));
  const size_t o_twn = o_twm + al(M * sizeof(float2));
  const size_t o_rows = o_twn + al(M * sizeof(float2));
  const size_t o_w = o_rows + al(p.n_mels * sizeof(MelRow));
  const size_t o_tbl = o_w + al(static_cast<size_t>(p.nnz > 0 ? p.nnz : 1) * sizeof(float));
  const size_t o_bw = o_tbl + al((8 + 4 * p.blocks.size()) * sizeof(int32_t));
  const size_t o_taps = o_bw + al(std::max<size_t>(p.blk_w.size(), 1) * sizeof(float));
  const size_t o_quad = o_taps + al(p.taps.size() * sizeof(BinTap));
  const size_t o_qw = o_quad + al((16 + p.quad_hdr.size()) * sizeof(int32_t));
  const size_t total = o_qw + al(std::max<size_t>(p.quad_w.size(), 1) * sizeof(float));
  // the kernels copy win2 and tw_p as one block of 16*M bytes
  if (o_twp != o_win + static_cast<size_t>(M) * sizeof(float2) && tables_in_lds(p.fft.n1, M))
    return set_error(FM_E_HIP, "internal: pass-1 tables are not contiguous");
  std::vector<unsigned char> host(total, 0);
  float* win2 = reinterpret_cast<float*>(host.data() + o_win);
  for (int j = 0; j < p.n_fft; ++j) win2[j] = 0.5f * p.window[j];  // exact scaling
  std::copy(p.tw_p.begin(), p.tw_p.end(), reinterpret_cast<float*>(host.data() + o_twp));
  std::copy(p.tw_m.begin(), p.tw_m.end(), reinterpret_cast<float*>(host.data() + o_twm));
  std::copy(p.tw_n.begin(), p.tw_n.end(), reinterpret_cast<float*>(host.data() + o_twn));
  std::copy(p.rows.begin(), p.rows.end(), reinterpret_cast<MelRow*>(host.data() + o_rows));
  std::copy(p.mel_w.begin(), p.mel_w.end(), reinterpret_cast<float*>(host.data() + o_w));
  int32_t* tbl = reinterpret_cast<int32_t*>(host.data() + o_tbl);
  for (int w = 0; w <= kMelWaves; ++w) tbl[w] = p.wave_beg[w];
  for (size_t j = 0; j < p.blocks.size(); ++j) {
    tbl[8 + 4 * j + 0] = p.blocks[j].kb;
    tbl[8 + 4 * j + 1] = mel_step_word(p.blocks[j].ksteps, p.blocks[j].s_hi);
    tbl[8 + 4 * j + 2] = p.blocks[j].w_off;
    tbl[8 + 4 * j + 3] = mel_filter_word(p.blocks[j].mel0, p.blocks[j].nrow);
  }
  std::copy(p.blk_w.begin(), p.blk_w.end(), reinterpret_cast<float*>(host.data() + o_bw));
  std::copy(p.taps.begin(), p.taps.end(), reinterpret_cast<BinTap*>(host.data() + o_taps));
  int32_t* qt = reinterpret_cast<int32_t*>(host.data() + o_quad);
  for (int sh = 0; sh <= kMelShares; ++sh) qt[sh] = p.quad_beg[sh];
  std::copy(p.quad_hdr.begin(), p.quad_hdr.end(), qt + 16);
  std::copy(p.quad_w.begin(), p.quad_w.end(), reinterpret_cast<float*>(host.data() + o_qw));
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
  p.d_tw_p = base + o_twp;
  p.d_tw_m = base + o_twm;
  p.d_tw_n = base + o_twn;
  p.d_rows = base + o_rows;
  p.d_mel_w = base + o_w;
  p.d_mel_tbl = base + o_tbl;
  p.d_blk_w = base + o_bw;
  p.d_taps = base + o_taps;
  p.d_quad = base + o_quad;
  p.d_quad_w = base + o_qw;
  // The large-FFT kernel: LDS opt-in and residency (no other kernel).
  if (p.lfft.n3) {  // the three-pass kernel (n_fft 8192, 16384; 4096 beside the split one)
    for (int dt : {FM_F32, FM_I16}) {
      void* k = select_large_kernel(p, dt);
      if (!k) return set_error(FM_E_UNSUPPORTED, "no large-FFT kernel for this n_fft");
      e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, p.large_lds);
      if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (large)");
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, select_large_kernel(p, FM_F32), p.large_threads,
                                                     p.large_lds) == hipSuccess)
      p.large_wg_per_cu = std::max(1, n);
  }
  if (p.fwd_variant == kFwdLarge) {
    p.has_device = true;
    return FM_OK;
  }
  // Tiles above 64 KB of LDS need the per-kernel opt-in (every variant a
  // call may choose: gather or tile copy, pair or row layout).
  const bool rows_built = p.fwd_variant == kFwdRows || p.fwd_variant == kFwdAuto;
  for (int dt : {FM_F32, FM_I16}) {
    for (bool copy : {false, true}) {
      for (bool rows : {false, true}) {
        for (bool prio : {false, true}) {
          if ((rows && !rows_built) || (prio && !copy)) continue;
          void* k = select_kernel(p, dt, copy, rows, prio);
          if (!k) return set_error(FM_E_UNSUPPORTED, "no kernel for this n_fft");
          e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
          if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
        }
      }
    }
  }
  // The paired kernel: LDS opt-in and residency.
  if (p.fwd_variant == kFwdPaired) {
    for (int dt : {FM_F32, FM_I16}) {
      void* k = select_pair_kernel(p, dt);
      if (!k) return set_error(FM_E_UNSUPPORTED, "no paired kernel for this n_fft");
      e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, p.pair_lds_bytes);
      if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (paired)");
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, select_pair_kernel(p, FM_F32), kPairThreads,
                                                     p.pair_lds_bytes) == hipSuccess)
      p.pair_wg_per_cu = std::max(1, n);
  }
  // Resident workgroups per CU for each tile size (registers and LDS).
  p.wg_per_cu.assign(p.tile_max + 1, 1);
  if (void* k = select_kernel(p, FM_F32, false, false)) {
    for (int g = (p.tile_max + 1) / 2; g <= p.tile_max; ++g) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, p.threads, tile_lds_bytes(p, g, false)) == hipSuccess)
        p.wg_per_cu[g] = std::max(1, n);
    }
  }
  // The row layout (same LDS layout): residency.
  if (rows_built) {
    p.rows_wg_per_cu.assign(p.tile_max + 1, 1);
    void* k = select_kernel(p, FM_F32, false, true);
    for (int g = (p.tile_max + 1) / 2; g <= p.tile_max; ++g) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kRowsThreads, tile_lds_bytes(p, g, true)) == hipSuccess)
        p.rows_wg_per_cu[g] = std::max(1, n);
    }
  }
  // The backward kernel of the plan's power mode: LDS opt-in and residency.
  p.bwd_wg_per_cu.assign(p.bwd_chunk_max + 1, 1);
  if (p.bwd_chunk_max > 0) {
    void* kb = select_backward_kernel(p);
    if (!kb) return set_error(FM_E_UNSUPPORTED, "no backward kernel for this n_fft");
    e = hipFuncSetAttribute(kb, hipFuncAttributeMaxDynamicSharedMemorySize, kBwdLdsMax);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute (backward)");
    for (int c = 1; c <= p.bwd_chunk_max; ++c) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kb, kBwdThreads, bwd_lds_bytes(p, c)) == hipSuccess)
        p.bwd_wg_per_cu[c] = std::max(1, n);
    }
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
                   void* out, void* stream) {
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
  const FwdChoice c = choose_forward(p, batch, T);
  if (c.variant == kFwdPaired) {
    if (length > (1 << 29)) return set_error(FM_E_INVAL, "problem too large for one launch (length <= 2^29)");
    const int64_t total = batch * T;
    const int64_t grid = c.workgroups;
    PArgs a;
    a.in = in;
    a.out = out;
    a.win = static_cast<const float*>(p.d_win2);
    a.tw_n = static_cast<const float2*>(p.d_tw_n);
    a.mel_tbl = static_cast<const int*>(p.d_mel_tbl);
    a.blk_w = static_cast<const float*>(p.d_blk_w);
    a.length = length;
    a.in_elems = batch * length;
    a.total = total;
    a.n_frames = static_cast<int>(T);
    a.hop = p.hop;
    a.pad = p.pad_left + p.zpad;
    a.zpad = p.zpad;
    a.pad_mode = p.pad_mode;
    a.n_mels = p.n_mels;
    a.chunk = p.pair_chunk;
    a.w_floats = static_cast<int>(p.blk_w.size());
    a.out_f16 = p.out_dtype == FM_F16 ? 1 : 0;
    a.half_power = static_cast<float>(p.power * 0.5);
    a.span_lds = p.pair_span_lds;
    a.w_lds = p.pair_w_lds;
    void* k = select_pair_kernel(p, in_dtype);
    if (!k) return set_error(FM_E_UNSUPPORTED, "no paired kernel for this n_fft");
    void* args[] = {&a};
    e = hipLaunchKernel(k, dim3(static_cast<unsigned>(grid)), dim3(kPairThreads), args,
                        static_cast<size_t>(p.pair_lds_bytes), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kernel launch (paired)");
    return FM_OK;
  }
  if (c.variant == kFwdLarge) {
    if (length > (1 << 29)) return set_error(FM_E_INVAL, "problem too large for one launch (length <= 2^29)");
    const int64_t g = c.tile;
    const int64_t tiles = (T + g - 1) / g;
    if (tiles * batch > INT32_MAX) return set_error(FM_E_INVAL, "problem too large for one launch");
    LArgs a;
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
    a.pad = p.pad_left + p.zpad;
    a.zpad = p.zpad;
    a.n_mels = p.n_mels;
    a.tile = static_cast<int>(g);
    a.tiles_per_signal = static_cast<int>(tiles);
    a.pad_mode = p.pad_mode;
    a.half_power = static_cast<float>(p.power * 0.5);
    const size_t esz = (in_dtype == FM_I16) ? 2 : 4;
    const uintptr_t ia = reinterpret_cast<uintptr_t>(in);
    a.vec_ok = (ia % (2 * esz) == 0) && (length % 2 == 0) && (p.hop % 2 == 0) &&
               ((p.pad_left + p.zpad) % 2 == 0);
    a.out_f16 = p.out_dtype == FM_F16 ? 1 : 0;
    a.w16 = (p.nnz + 3) / 4;
    a.w_lds = large_exchange_bytes(p.lfft.n1, p.lfft.n2, p.lfft.n3);
    void* k = select_large_kernel(p, in_dtype);
    if (!k) return set_error(FM_E_UNSUPPORTED, "no large-FFT kernel for this n_fft");
    void* args[] = {&a};
    e = hipLaunchKernel(k, dim3(static_cast<unsigned>(tiles * batch)), dim3(p.large_threads), args,
                        static_cast<size_t>(p.large_lds), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kernel launch (large)");
    return FM_OK;
  }
  const bool rows = c.variant == kFwdRows;
  const int G = c.tile;
  const int64_t tiles = (T + G - 1) / G;
  if (length > (1 << 29) || tiles * batch > INT32_MAX)
    return set_error(FM_E_INVAL, "problem too large for one launch (length <= 2^29, tiles < 2^31)");
  const int lds = tile_lds_bytes(p, G, rows);
  const int64_t n_tiles = tiles * batch;

  KArgs a;
  a.in = in;
  a.out = out;
  a.win2 = static_cast<const float2*>(p.d_win2);
  a.tw_m = static_cast<const float2*>(p.d_tw_p);
  a.tw_n = static_cast<const float2*>(p.d_tw_n);
  a.length = length;
  a.n_frames = static_cast<int>(T);
  a.hop = p.hop;
  a.pad = p.pad_left + p.zpad;
  a.zpad = p.zpad;
  a.n_mels = p.n_mels;
  a.tile = G;
  a.tiles_per_signal = static_cast<int>(tiles);
  a.pad_mode = p.pad_mode;
  a.half_power = static_cast<float>(p.power * 0.5);
  const size_t esz = (in_dtype == FM_I16) ? 2 : 4;
  const uintptr_t ia = reinterpret_cast<uintptr_t>(in);
  a.vec_ok = (ia % (2 * esz) == 0) && (length % 2 == 0) && (p.hop % 2 == 0) &&
             ((p.pad_left + p.zpad) % 2 == 0);
  a.mel_tbl = static_cast<const int*>(p.d_mel_tbl);
  a.blk_w = static_cast<const float*>(p.d_blk_w);
  // wide tiles project on the vector units (no block weights to copy)
  a.mel_valu = tile_mel_valu(p, G) ? 1 : 0;
  a.w_chunks = (p.w_in_lds && !a.mel_valu) ? static_cast<int>(p.blk_w.size() / 256) : 0;
  a.w_lds = tile_weights_offset(p, G);
  a.quad_tbl = static_cast<const int*>(p.d_quad);
  a.quad_w = static_cast<const float*>(p.d_quad_w);
  a.out_f16 = p.out_dtype == FM_F16 ? 1 : 0;
  a.tab_lds = tile_tables_offset(p, G);
  a.twn_lds = tile_twiddles_offset(p, G, rows);

  void* k = select_kernel(p, in_dtype, c.copy, rows, c.phase_prio && c.copy);
  if (!k) return set_error(FM_E_UNSUPPORTED, "no kernel for this n_fft");
  void* args[] = {&a};
  e = hipLaunchKernel(k, dim3(static_cast<unsigned>(n_tiles)), dim3(rows ? kRowsThreads : p.threads),
                      args, static_cast<size_t>(lds), static_cast<hipStream_t>(stream));
  // (the launch's own status only: hipGetLastError would also report, and
  // clear, an unrelated earlier failure on the caller's thread)
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return FM_OK;
}

namespace {

// Frames per backward pass for this call.  A main workgroup recomputes the
// `halo` frames before its tile, so a pass of c frames advances c - halo;
// the cost model is the forward's (rounds of resident workgroups times a
// workgroup's pass-1 rounds plus a fixed part), ties to smaller passes.
int choose_bwd_chunk(const Plan& p, int64_t batch, int64_t T, int halo, int64_t n_edge) {
  if (p.bwd_chunk_override > halo) return p.bwd_chunk_override;
  const int ncu = p.n_cu > 0 ? p.n_cu : 256;
  const int slots = std::max(1, kBwdThreads / p.fft.n2);
  int best = p.bwd_chunk_max;
  int64_t best_cost = INT64_MAX;
  for (int c = halo + 1; c <= p.bwd_chunk_max; ++c) {
    const int g = c - halo;
    const int64_t wgs = batch * ((T + g - 1) / g) + n_edge;
    const int occ = p.bwd_wg_per_cu[c] > 0 ? p.bwd_wg_per_cu[c] : 1;
    const int64_t per_round = static_cast<int64_t>(ncu) * occ;
    const int64_t cost = (wgs + per_round - 1) / per_round * ((c + slots - 1) / slots + 4);
    if (cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

}  // namespace

int launch_backward(const Plan& p, const float* in, int64_t batch, int64_t length,
                    const float* grad_out, float* grad_in, void* stream) {
  if (!p.has_device) return set_error(FM_E_NODEVICE, "plan was built without device tables");
  if (batch < 0) return set_error(FM_E_INVAL, "batch must be >= 0");
  const int64_t T = out_frames(p, length);
  if (T < 0) return static_cast<int>(T);
  if (batch == 0) return FM_OK;
  if (!in || !grad_out || !grad_in) return set_error(FM_E_INVAL, "null input, gradient or output pointer");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != p.device) return set_error(FM_E_INVAL, "plan belongs to another device than the current one");
  if (length > (1 << 29)) return set_error(FM_E_INVAL, "problem too large for one launch (length <= 2^29)");
  const int halo = (p.n_fft - 1) / p.hop;
  const int edge = bwd_edge(p);
  const int whole = 2 * static_cast<int64_t>(edge) >= length ? 1 : 0;
  // head and tail zones in workgroups of their own, unless circular padding
  // sends tail frames' gradients to the head (or one zone covers the signal)
  const int edge_split = (edge > 0 && !whole && p.pad_mode != FM_PAD_CIRCULAR) ? 1 : 0;
  const int64_t n_edge = edge > 0 ? batch * (edge_split ? 2 : 1) : 0;
  // One pass per main workgroup when the overlap fits a pass; else tiles of
  // halo + 1 frames whose frames (2 halo + 1) take several passes, the owned
  // samples (at most tile*hop + n_fft + padding) accumulating in LDS.
  int chunk, tile, multi = 0, oacc = 0;
  if (p.bwd_chunk_max >= halo + 1) {
    chunk = choose_bwd_chunk(p, batch, T, halo, n_edge);
    tile = chunk - halo;
  } else {
    multi = 1;
    tile = halo + 1;
    oacc = tile * p.hop + p.n_fft + p.pad_left + p.zpad;
    chunk = p.bwd_chunk_max;
    while (chunk > 1 && bwd_lds_bytes(p, chunk) + 4L * oacc > kBwdLdsMax) --chunk;
    if (p.bwd_chunk_max < 1 || bwd_lds_bytes(p, chunk) + 4L * oacc > kBwdLdsMax)
      return set_error(FM_E_UNSUPPORTED, "backward: the samples one workgroup owns do not fit its LDS "
                                         "(hop " + std::to_string(p.hop) + ", n_fft " + std::to_string(p.n_fft) + ")");
  }
  const int64_t tiles = (T + tile - 1) / tile;
  const int64_t n_main = whole ? 0 : batch * tiles;
  if (n_main + n_edge > INT32_MAX) return set_error(FM_E_INVAL, "problem too large for one launch");

  BArgs a;
  a.in = in;
  a.gout = grad_out;
  a.gin = grad_in;
  a.win2 = static_cast<const float2*>(p.d_win2);
  a.tw_m = static_cast<const float2*>(p.d_tw_m);
  a.tw_n = static_cast<const float2*>(p.d_tw_n);
  a.taps = static_cast<const BinTap*>(p.d_taps);
  a.length = length;
  a.n_frames = static_cast<int>(T);
  a.hop = p.hop;
  a.pad = p.pad_left + p.zpad;
  a.zpad = p.zpad;
  a.pad_mode = p.pad_mode;
  a.n_mels = p.n_mels;
  a.tile = tile;
  a.halo = halo;
  a.tiles_per_signal = static_cast<int>(tiles);
  a.n_edge = static_cast<int>(n_edge);
  a.edge = edge;
  a.edge_split = edge_split;
  a.whole = whole;
  a.chunk = chunk;
  const uintptr_t ia = reinterpret_cast<uintptr_t>(in);
  a.vec_ok = (ia % 8 == 0) && (length % 2 == 0) && (p.hop % 2 == 0) && ((p.pad_left + p.zpad) % 2 == 0);
  a.multi = multi;
  a.oacc_off = bwd_lds_bytes(p, chunk) / 4;
  a.g_off = bwd_grad_offset(p, chunk);
  a.gt_off = bwd_gtile_offset(p, chunk);
  a.acc_off = bwd_acc_offset(p, chunk);
  a.power = static_cast<float>(p.power);
  a.half_power = static_cast<float>(p.power * 0.5);

  void* k = select_backward_kernel(p);
  if (!k) return set_error(FM_E_UNSUPPORTED, "no backward kernel for this n_fft");
  void* args[] = {&a};
  e = hipLaunchKernel(k, dim3(static_cast<unsigned>(n_main + n_edge)), dim3(kBwdThreads), args,
                      static_cast<size_t>(bwd_lds_bytes(p, chunk) + 4 * oacc), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  return FM_OK;
}

}  // namespace fm
