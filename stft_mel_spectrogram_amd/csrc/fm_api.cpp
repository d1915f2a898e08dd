// C ABI of the fused mel-spectrogram forward pass (declared in include/fm.h).
#include <cstring>
#include <new>
#include <string>

#include "fm_internal.h"

struct fm_plan {
  fm::Plan p;
};

namespace fm {

namespace {
thread_local std::string g_last_error;
}

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

const char* last_error_cstr() { return g_last_error.c_str(); }

}  // namespace fm

namespace {

int create(fm_plan** out, bool with_device, const fm_args* a) {
  if (!out) return fm::set_error(FM_E_INVAL, "out must not be NULL");
  *out = nullptr;
  if (!a) return fm::set_error(FM_E_INVAL, "args must not be NULL");
  fm_plan* h = new (std::nothrow) fm_plan();
  if (!h) return fm::set_error(FM_E_NOMEM, "host allocation failed");
  int st = fm::build_host_plan(h->p, *a);
  if (st == FM_OK && with_device) st = fm::upload_plan(h->p);
  if (st != FM_OK) {
    fm::free_plan_device(h->p);
    delete h;
    return st;
  }
  *out = h;
  return FM_OK;
}

fm_args positional(int sample_rate, int n_fft, int win_length, int hop_length, int n_mels,
                   double f_min, double f_max, double power, int center, int pad_mode,
                   int mel_scale, int norm) {
  fm_args a;
  fm::default_args(&a);
  a.sample_rate = sample_rate;
  a.n_fft = n_fft;
  a.win_length = win_length;
  a.hop_length = hop_length;
  a.n_mels = n_mels;
  a.f_min = f_min;
  a.f_max = f_max;
  a.power = power;
  a.center = center;
  a.pad_mode = pad_mode;
  a.mel_scale = mel_scale;
  a.norm = norm;
  return a;
}

}  // namespace

extern "C" {

int fm_args_default(fm_args* args) {
  if (!args) return fm::set_error(FM_E_INVAL, "args must not be NULL");
  fm::default_args(args);
  return FM_OK;
}

int fm_plan_create_args(fm_plan** out, const fm_args* args) { return create(out, true, args); }

int fm_plan_create_args_host(fm_plan** out, const fm_args* args) {
  return create(out, false, args);
}

int fm_plan_create(fm_plan** out, int sample_rate, int n_fft, int win_length, int hop_length,
                   int n_mels, double f_min, double f_max, double power, int center, int pad_mode,
                   int mel_scale, int norm) {
  const fm_args a = positional(sample_rate, n_fft, win_length, hop_length, n_mels, f_min, f_max,
                              power, center, pad_mode, mel_scale, norm);
  return create(out, true, &a);
}

int fm_plan_create_host(fm_plan** out, int sample_rate, int n_fft, int win_length,
                        int hop_length, int n_mels, double f_min, double f_max, double power,
                        int center, int pad_mode, int mel_scale, int norm) {
  const fm_args a = positional(sample_rate, n_fft, win_length, hop_length, n_mels, f_min, f_max,
                              power, center, pad_mode, mel_scale, norm);
  return create(out, false, &a);
}

int fm_forward(const fm_plan* plan, const void* in, int in_dtype, int64_t batch, int64_t length,
               void* out, void* stream) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  return fm::launch_forward(plan->p, in, in_dtype, batch, length, out, stream);
}

int fm_backward(const fm_plan* plan, const float* in, int64_t batch, int64_t length,
                const float* grad_out, float* grad_in, void* stream) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  return fm::launch_backward(plan->p, in, batch, length, grad_out, grad_in, stream);
}

int fm_forward_config(const fm_plan* plan, int64_t batch, int64_t length, int* variant,
                      int* tile_frames, int64_t* workgroups) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  if (batch < 0) return fm::set_error(FM_E_INVAL, "batch must be >= 0");
  const int64_t T = fm::out_frames(plan->p, length);
  if (T < 0) return static_cast<int>(T);
  const fm::FwdChoice c = fm::choose_forward(plan->p, batch, T);
  if (variant) *variant = c.variant;
  if (tile_frames) *tile_frames = c.tile;
  if (workgroups) *workgroups = c.workgroups;
  return FM_OK;
}

int64_t fm_out_frames(const fm_plan* plan, int64_t length) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  return fm::out_frames(plan->p, length);
}

int fm_plan_destroy(fm_plan* plan) {
  if (!plan) return FM_OK;
  fm::free_plan_device(plan->p);
  delete plan;
  return FM_OK;
}

const char* fm_strerror(int status) {
  switch (status) {
    case FM_OK: return "success";
    case FM_E_INVAL: return "invalid argument";
    case FM_E_UNSUPPORTED: return "unsupported configuration";
    case FM_E_HIP: return "HIP runtime error";
    case FM_E_NOMEM: return "out of memory";
    case FM_E_NODEVICE: return "plan has no device tables";
    default: return "unknown status";
  }
}

const char* fm_last_error(void) { return fm::last_error_cstr(); }

int fm_plan_info_get(const fm_plan* plan, fm_plan_info* info) {
  if (!plan || !info) return fm::set_error(FM_E_INVAL, "plan and info must not be NULL");
  const fm::Plan& p = plan->p;
  info->n_fft = p.n_fft;
  info->win_length = p.win_length;
  info->hop_length = p.hop;
  info->n_mels = p.n_mels;
  info->n_freqs = p.n_freqs;
  info->pad = p.zpad;
  info->normalized = p.normalized;
  info->out_dtype = p.out_dtype;
  info->nnz = p.nnz;
  info->w_max = p.w_max;
  info->fft_n1 = p.fft.n1;
  info->fft_n2 = p.fft.n2;
  info->fft_n3 = p.fft.n3;
  const bool paired = p.fwd_variant == fm::kFwdPaired;
  info->tile_frames = paired ? p.pair_chunk : p.tile_max;
  info->threads = paired ? fm::kPairThreadsHost
                         : (p.fwd_variant == fm::kFwdRows ? fm::kRowsThreads : p.threads);
  info->lds_bytes = paired ? p.pair_lds_bytes : p.lds_bytes;
  info->forward_variant = p.fwd_variant;
  info->has_device = p.has_device ? 1 : 0;
  return FM_OK;
}

int fm_plan_tables(const fm_plan* plan, float* window, int32_t* mel_first, int32_t* mel_len,
                   int32_t* mel_off, float* mel_w, float* tw_m, float* tw_n) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  const fm::Plan& p = plan->p;
  if (window) std::memcpy(window, p.window.data(), p.window.size() * sizeof(float));
  for (int m = 0; m < p.n_mels; ++m) {
    if (mel_first) mel_first[m] = p.rows[m].first;
    if (mel_len) mel_len[m] = p.rows[m].len;
    if (mel_off) mel_off[m] = p.rows[m].off;
  }
  if (mel_w && p.nnz) std::memcpy(mel_w, p.mel_w.data(), p.mel_w.size() * sizeof(float));
  if (tw_m) std::memcpy(tw_m, p.tw_m.data(), p.tw_m.size() * sizeof(float));
  if (tw_n) std::memcpy(tw_n, p.tw_n.data(), p.tw_n.size() * sizeof(float));
  return FM_OK;
}

int fm_plan_mel_blocks(const fm_plan* plan, int32_t* blocks, int32_t* wave_beg, float* weights,
                       int32_t* n_blocks, int64_t* n_weights) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  const fm::Plan& p = plan->p;
  if (blocks)
    for (size_t j = 0; j < p.blocks.size(); ++j) {
      blocks[4 * j + 0] = p.blocks[j].kb;
      blocks[4 * j + 1] = p.blocks[j].ksteps;
      blocks[4 * j + 2] = p.blocks[j].w_off;
      blocks[4 * j + 3] = fm::mel_filter_word(p.blocks[j].mel0, p.blocks[j].nrow);
    }
  if (wave_beg)
    for (int w = 0; w <= fm::kMelWaves; ++w) wave_beg[w] = p.wave_beg[w];
  if (weights) std::memcpy(weights, p.blk_w.data(), p.blk_w.size() * sizeof(float));
  if (n_blocks) *n_blocks = static_cast<int32_t>(p.blocks.size());
  if (n_weights) *n_weights = static_cast<int64_t>(p.blk_w.size());
  return FM_OK;
}

int fm_plan_mel_quads(const fm_plan* plan, int32_t* headers, int32_t* share_beg, float* weights,
                      int32_t* n_quads, int64_t* n_weights) {
  if (!plan) return fm::set_error(FM_E_INVAL, "plan must not be NULL");
  const fm::Plan& p = plan->p;
  const size_t nq = p.quad_hdr.size() / fm::kQuadHdr;
  if (headers)
    for (size_t q = 0; q < nq; ++q)
      for (int i = 0; i < 6; ++i) headers[6 * q + i] = p.quad_hdr[fm::kQuadHdr * q + i];
  if (share_beg)
    for (int s = 0; s <= fm::kMelShares; ++s) share_beg[s] = p.quad_beg[s];
  if (weights) std::memcpy(weights, p.quad_w.data(), p.quad_w.size() * sizeof(float));
  if (n_quads) *n_quads = static_cast<int32_t>(nq);
  if (n_weights) *n_weights = static_cast<int64_t>(p.quad_w.size());
  return FM_OK;
}

}  // extern "C"
