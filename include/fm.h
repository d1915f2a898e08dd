/*
 * fm.h -- C ABI of the fused mel-spectrogram forward pass for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the one the flashmel 0.1.0 page (PyPI sdist diff view)
 * describes: a torchaudio-MelSpectrogram-compatible forward pass -- centre
 * padding, framing at hop_length, periodic Hann window, real-to-complex FFT of
 * size n_fft, |X|^power and a projection onto a sparse triangular mel
 * filterbank -- in a single kernel launch (README "How it works"; argument
 * list and shape contract in README "Usage"; window and filterbank packing in
 * flashmel/filters.py).
 *
 * Conventions for every entry point:
 *   - Return value: FM_OK (0) on success, a negative FM_E_* code otherwise.
 *     On failure a message is kept per thread; fm_last_error() returns it.
 *   - Pointers named `in`/`out` are DEVICE pointers owned by the caller.
 *     Plans own their device tables; fm_plan_destroy frees them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Nothing here synchronises the device; fm_forward only enqueues.
 */
#ifndef FM_H_
#define FM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define FM_OK 0
#define FM_E_INVAL (-1)       /* invalid argument (bad value, null pointer)  */
#define FM_E_UNSUPPORTED (-2) /* valid for torchaudio, not built here         */
#define FM_E_HIP (-3)         /* a HIP runtime call failed                    */
#define FM_E_NOMEM (-4)       /* host or device allocation failed            */
#define FM_E_NODEVICE (-5)    /* plan has no device tables (host-only plan)  */

/* ---- enumerations -------------------------------------------------------- */
/* pad_mode: how frames read beyond the signal when center != 0 (README "How
 * it works": all four pad modes are index arithmetic).                      */
#define FM_PAD_REFLECT 0   /* x[-i] = x[i], edge sample not repeated         */
#define FM_PAD_CONSTANT 1  /* zeros                                          */
#define FM_PAD_REPLICATE 2 /* edge sample repeated                           */
#define FM_PAD_CIRCULAR 3  /* periodic wrap                                  */

/* mel_scale and norm: passed through to the filterbank construction
 * (flashmel/filters.py pack_fbank).                                        */
#define FM_MEL_HTK 0
#define FM_MEL_SLANEY 1
#define FM_NORM_NONE 0
#define FM_NORM_SLANEY 1

/* sample types.  Input: float32, or int16 PCM that the kernel multiplies by
 * 2^-15 as it loads it (README "Usage" lists both input types and that
 * scale).  Output: float32, or float16 (README "Usage", out_dtype): the
 * float32 result rounded to nearest at the store; values past 65504 become
 * inf.                                                                     */
#define FM_F32 0
#define FM_I16 1
#define FM_F16 2

/* normalized: STFT normalisation folded into the window (flashmel/filters.py
 * make_window): none, divide by sqrt(sum of the squared window), or divide
 * by sqrt(win_length).                                                     */
#define FM_NORMALIZED_NONE 0
#define FM_NORMALIZED_WINDOW 1
#define FM_NORMALIZED_FRAME_LENGTH 2

typedef struct fm_plan fm_plan;

/*
 * fm_args -- every argument of a plan (torchaudio MelSpectrogram's, README
 * "Usage", plus the output type).  Fill it with fm_args_default, which sets
 * torchaudio's defaults for n_fft = 400 at 16 kHz, then change fields.
 *   sample_rate, n_fft, win_length, hop_length, n_mels, f_min, f_max, power,
 *   center, pad_mode, mel_scale, norm: as for fm_plan_create below;
 *   pad        >= 0 zero samples added on both sides of the signal before the
 *              centre padding (which then reflects / repeats / wraps the
 *              zero-extended signal); at most 2^28;
 *   normalized FM_NORMALIZED_*;
 *   out_dtype  FM_F32 or FM_F16: the element type fm_forward writes.
 */
typedef struct fm_args {
  int sample_rate, n_fft, win_length, hop_length, n_mels;
  double f_min, f_max, power;
  int center, pad_mode, mel_scale, norm;
  int pad, normalized, out_dtype;
} fm_args;

/* sample_rate 16000, n_fft 400, win_length 400, hop_length 200, n_mels 128,
 * f_min 0, f_max 8000, power 2, center 1, reflect, HTK, no norm, pad 0, not
 * normalized, f32 output.  FM_E_INVAL if args is NULL.                      */
int fm_args_default(fm_args* args);

/*
 * fm_plan_create_args / fm_plan_create_args_host -- fm_plan_create and
 * fm_plan_create_host with every argument in one struct (read, not kept).
 * Same ownership, validation and errors; a plan made with out_dtype FM_F16
 * writes float16 from fm_forward.
 */
int fm_plan_create_args(fm_plan** out, const fm_args* args);
int fm_plan_create_args_host(fm_plan** out, const fm_args* args);

/*
 * fm_plan_create -- build a plan on the CURRENT HIP device.
 *
 * Arguments are torchaudio MelSpectrogram's (README "Usage"):
 *   sample_rate > 0; n_fft 400 or a power of two from 64 to 16384 (others:
 *   FM_E_UNSUPPORTED; README "Usage" allows exactly these);
 *   0 < win_length <= n_fft (a shorter window is zero-padded centred,
 *   flashmel/filters.py make_window); hop_length > 0;
 *   1 <= n_mels <= 256 (README "Usage");
 *   0 <= f_min < f_max <= sample_rate/2;  power > 0 (2: power spectrum,
 *   1: magnitude);  center 0/1;  pad_mode FM_PAD_*;  mel_scale FM_MEL_*;
 *   norm FM_NORM_*.
 *
 * The window, the CSR filterbank (per mel: first bin, run length, offset,
 * weights), the FFT twiddle tables and the tile geometry are built in
 * float64 on the host, rounded once to float32 and uploaded.  *out receives
 * a plan that owns that device memory; it is immutable and may be used
 * concurrently from several streams of the same device.
 *
 * Errors: FM_E_INVAL / FM_E_UNSUPPORTED for arguments, FM_E_NOMEM,
 * FM_E_HIP (no device, upload failed).  *out is set to NULL on failure.
 */
int fm_plan_create(fm_plan** out, int sample_rate, int n_fft, int win_length,
                   int hop_length, int n_mels, double f_min, double f_max,
                   double power, int center, int pad_mode, int mel_scale,
                   int norm);

/*
 * fm_plan_create_host -- same arguments and validation as fm_plan_create,
 * but builds only the host tables and touches no GPU.  Such a plan serves
 * fm_plan_info / fm_plan_tables / fm_out_frames; fm_forward on it returns
 * FM_E_NODEVICE.
 */
int fm_plan_create_host(fm_plan** out, int sample_rate, int n_fft,
                        int win_length, int hop_length, int n_mels,
                        double f_min, double f_max, double power, int center,
                        int pad_mode, int mel_scale, int norm);

/*
 * fm_forward -- enqueue one mel-spectrogram forward pass on `stream`.
 *
 * The flashmel 0.1.0 page, README "Usage", defines the call: a batch of
 * signals (..., time) in float32 or int16 on the GPU gives (..., n_mels,
 * n_frames), e.g. [8, 480000] at hop 160 gives [8, 128, 3001]; README "How
 * it works" puts the whole chain (padding as index arithmetic, window, real
 * FFT, |X|^power, sparse mel projection) in one kernel launch.  Here the
 * leading dimensions are flattened into `batch`.
 *
 *   in     device pointer to [batch, length] samples, row-major, contiguous,
 *          of type in_dtype (FM_F32: float, FM_I16: int16_t).
 *   out    device pointer to [batch, n_mels, n_frames] elements of the plan's
 *          out_dtype (float32 unless made with FM_F16: float16), row-major,
 *          contiguous (frames fastest), n_frames = fm_out_frames(plan,
 *          length), aligned to its element size.  Every element is written.
 *   batch  >= 0 (0 is a no-op); length >= 1, and with center + reflect
 *          padding length + 2*pad > n_fft/2 (a single reflection), with
 *          circular padding length + 2*pad >= n_fft/2, otherwise FM_E_INVAL;
 *          without center length + 2*pad >= n_fft.
 *
 * One kernel launch; no allocation, no synchronisation.  Launch errors are
 * reported as FM_E_HIP.  The plan must live on the device that is current.
 */
int fm_forward(const fm_plan* plan, const void* in, int in_dtype,
               int64_t batch, int64_t length, void* out, void* stream);

/*
 * fm_backward -- enqueue the gradient of the forward pass with respect to
 * its float32 input: grad_in = d/dx sum(grad_out * mel(x)).
 *
 * The flashmel 0.1.0 page (README "Usage") leaves the transform
 * inference-only; the specux "Backends" page (section "Gradients") computes
 * a spectrogram's gradient as the analytic adjoint, in kernels of the same
 * family as the forward, with a bitwise-reproducible mode.  This entry point
 * applies that adjoint, always deterministically: the transposed filterbank, the gradient of |X|^power
 * (p |X|^(p-2) X, taken as 0 where X = 0 and power != 2), the adjoint of
 * the one-sided DFT (an inverse real FFT), the window, overlap-add of the
 * frames, and the adjoint of the padding (gradients of padded positions go
 * to the samples they copy).
 *
 *   in        device pointer to the forward input [batch, length], float32,
 *             row-major, contiguous (the spectrum is recomputed from it).
 *   grad_out  device pointer to [batch, n_mels, n_frames] float32 (whatever
 *             the plan's out_dtype), n_frames = fm_out_frames(plan, length).
 *   grad_in   device pointer to [batch, length] float32; every element is
 *             written (not accumulated).  Must not overlap the inputs.
 *   batch, length  as for fm_forward.
 *
 * Any hop: when more frames overlap one sample than one workgroup pass
 * holds, the workgroups take several passes.  FM_E_UNSUPPORTED for n_fft
 * 8192 and 16384 (no backward kernel is built for them), and when the
 * samples one workgroup owns (2 n_fft + 2 pad floats or so) do not fit its
 * LDS next to one frame's pass (a very large `pad`).  One kernel launch; no
 * allocation, no synchronisation.
 */
int fm_backward(const fm_plan* plan, const float* in, int64_t batch, int64_t length,
                const float* grad_out, float* grad_in, void* stream);

/*
 * fm_out_frames -- frames per signal for a given length (L = length + 2*pad),
 * the last dimension of fm_forward's output (README "Usage": the output
 * shape (..., n_mels, n_frames), 480000 samples at hop 160 giving 3001):
 *   center: 1 + floor(L / hop) for even n_fft (generally
 *           1 + floor((L + 2*(n_fft/2) - n_fft) / hop));
 *   else:   1 + floor((L - n_fft) / hop).
 * Returns a negative FM_E_* code if the length is invalid for the plan.
 */
int64_t fm_out_frames(const fm_plan* plan, int64_t length);

/*
 * fm_forward_config -- how fm_forward runs a call of `batch` signals of
 * `length` samples on this plan, without running it: *variant = the kernel
 * (FM_FWD_SPLIT, FM_FWD_ROWS, FM_FWD_PAIRED or FM_FWD_LARGE; never
 * FM_FWD_AUTO), *tile_frames = frames per workgroup tile (PAIRED: frames per
 * chunk at most), *workgroups = workgroups launched (0 for batch 0).  The
 * choice depends on the device the plan was created on (its compute units
 * and the kernels' residency); a host-only plan assumes 256 compute units
 * and one resident workgroup per unit.  Any output pointer may be NULL.
 * Returns FM_OK, FM_E_INVAL (NULL plan, batch < 0) or the negative code of
 * an invalid length (as fm_out_frames).  Operation-wise this is a host-side
 * query of the launch geometry behind the pages' one-launch forward pass
 * (flashmel 0.1.0 README "How it works").
 */
int fm_forward_config(const fm_plan* plan, int64_t batch, int64_t length, int* variant,
                      int* tile_frames, int64_t* workgroups);

/* fm_plan_destroy -- free the plan and its device tables.  NULL is a no-op. */
int fm_plan_destroy(fm_plan* plan);

/* Human-readable text for a status code (static storage).                 */
const char* fm_strerror(int status);

/* Message of the last failure on this thread ("" if none).                */
const char* fm_last_error(void);

/* ---- host-side inspection (used by CPU tests; no GPU needed) ------------ */

typedef struct fm_plan_info {
  int n_fft, win_length, hop_length, n_mels, n_freqs; /* n_freqs = n_fft/2+1 */
  int pad, normalized, out_dtype;
  int nnz;          /* nonzero filterbank weights (CSR length)              */
  int w_max;        /* widest filter (bins)                                 */
  int fft_n1, fft_n2; /* complex FFT of n_fft/2 = fft_n1 * fft_n2 points of
                       the split forward kernel and of the backward          */
  int tile_frames;  /* frames per workgroup tile (paired: per chunk)        */
  int threads;      /* threads per workgroup (FM_FWD_AUTO: of the split
                       kernel; the row kernel runs 512)                    */
  int lds_bytes;    /* dynamic LDS per workgroup                            */
  int has_device;   /* 1 if the plan owns device tables                     */
  int forward_variant; /* FM_FWD_SPLIT, FM_FWD_PAIRED, FM_FWD_LARGE,
                          FM_FWD_ROWS or FM_FWD_AUTO                       */
  int fft_n3;       /* FM_FWD_LARGE: n_fft/2 = fft_n1 * fft_n2 * fft_n3 (three
                       passes); 0 otherwise                                  */
} fm_plan_info;

/* Forward kernel variants.  SPLIT: each frame's real FFT through a complex
 * FFT of n_fft/2 points and the real-spectrum split, one tile of frames per
 * workgroup.  PAIRED: two frames per complex FFT of n_fft points (the
 * pages' packing of two real frames into one complex transform, README "How
 * it works"), persistent workgroups that walk their frames in chunks and load
 * the next chunk while transforming the current one; built for n_fft = 400,
 * taken only when the environment variable FM_FORWARD=paired is set at plan
 * creation (measured slower than SPLIT; kept for A/B measurements).
 * LARGE: n_fft 8192 and 16384, whose complex FFT of n_fft/2 points runs in
 * three passes over one LDS buffer, one frame at a time per workgroup, with
 * the mel projection over the CSR rows (these sizes have no backward).  A
 * SPLIT plan of n_fft 4096 also holds this kernel
 * (2048 = 16 x 16 x 8) and runs a call on it when the SPLIT tiles would
 * outnumber the compute units (fm_forward_config reports LARGE then; the
 * plan's own shape, its info and its backward stay SPLIT); FM_FORWARD=large
 * or split at plan creation forces the choice.
 * ROWS: the SPLIT chain with 512-thread workgroups whose second FFT pass
 * gives each row of fft_n2 points of a frame its own thread (the mirrored
 * row's values exchanged between lanes); built for n_fft 64 ... 2048.
 * AUTO (the default for n_fft 64 ... 2048): ROWS or SPLIT chosen per call
 * from the call's size (fm_forward_config reports the choice):
 * n_fft 256, 400, 512 and 2048 always ROWS; the other sizes ROWS when its
 * workgroups number at most the device's compute units.  FM_FORWARD=rows or
 * FM_FORWARD=split at plan creation forces one of them.  ROWS and SPLIT
 * compute the same operations in the same order: their outputs are
 * identical.                                                             */
#define FM_FWD_SPLIT 0
#define FM_FWD_PAIRED 1
#define FM_FWD_LARGE 2
#define FM_FWD_ROWS 3
#define FM_FWD_AUTO 4

int fm_plan_info_get(const fm_plan* plan, fm_plan_info* info);

/*
 * fm_plan_tables -- copy the host tables of a plan.  Any pointer may be NULL
 * to skip that table.  Sizes: window[n_fft] (float32, with the plan's
 * normalisation; the device copy is further scaled by 1/2 for the real-FFT
 * post-processing);
 * mel_first[n_mels], mel_len[n_mels], mel_off[n_mels] (int32; CSR rows,
 * len 0 for an empty filter); mel_w[nnz] (float32);
 * tw_m[2*(n_fft/2)] interleaved re,im of exp(-2*pi*i*j/(n_fft/2));
 * tw_n[2*(n_fft/2)] interleaved re,im of exp(-2*pi*i*k/n_fft).
 */
int fm_plan_tables(const fm_plan* plan, float* window, int32_t* mel_first,
                   int32_t* mel_len, int32_t* mel_off, float* mel_w,
                   float* tw_m, float* tw_n);

/*
 * fm_plan_mel_blocks -- the mel stage's layout on the matrix cores (host
 * copy, for tests).  The filterbank is cut into blocks of up to 16
 * consecutive filters (16, and the longest blocks split into halves of
 * filters); block j covers bins kb .. kb + 4*ksteps - 1 and its weights are
 * stored dense, 64 floats per 4-bin step, float s*64 + l holding filter
 * mel0 + l%16 at bin kb + 4*s + l/16 (0 outside the filter, and for l%16 >=
 * nrow, the block's filter count).
 *   blocks[4*n_blocks]  int32 {kb, ksteps, w_off, mel0 + 65536*nrow} per
 *                       block, grouped by the workgroup wave that computes
 *                       them;
 *   wave_beg[5]         wave w computes blocks wave_beg[w] .. wave_beg[w+1]-1;
 *   weights[n_weights]  every block's weights (w_off indexes them), plus
 *                       zero slack at the end.
 * Any pointer may be NULL; call once with NULL arrays to learn the sizes.
 */
int fm_plan_mel_blocks(const fm_plan* plan, int32_t* blocks, int32_t* wave_beg,
                       float* weights, int32_t* n_blocks, int64_t* n_weights);

/*
 * fm_plan_mel_quads -- the mel stage's layout on the vector units (host copy,
 * for tests; the same projection as the blocks above, used by tiles of 17
 * frames or more).  Filters in quads of 4 consecutive filters (quad q: filters
 * 4q .. 4q+3, those past n_mels empty); a quad runs L steps of one bin, filter
 * a of the quad over bins start_a .. start_a + L - 1, weight w[4*(off + i) + a]
 * at step i (0 outside the filter).
 *   headers[6*n_quads]   int32 {start_0, start_1, start_2, start_3, L, off}
 *                        per quad;
 *   share_beg[9]         share s holds quads share_beg[s] .. share_beg[s+1]-1
 *                        (a workgroup of w waves gives each wave 8/w shares);
 *   weights[n_weights]   every quad's weights, 4 per step.
 * Any pointer may be NULL; call once with NULL arrays to learn the sizes.
 */
int fm_plan_mel_quads(const fm_plan* plan, int32_t* headers, int32_t* share_beg,
                      float* weights, int32_t* n_quads, int64_t* n_weights);

#ifdef __cplusplus
}
#endif

#endif /* FM_H_ */
