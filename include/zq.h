/*
 * zq.h -- C-ABI of libzq.so: weight-only quantized linear layers on AMD MI355X
 * (gfx950, CDNA4).
 *
 * The operation: Y[M][N] = X[M][K] * dequant(Wq)[N][K]^T, with fp16 or bf16
 * activations X, packed signed integer weight codes Wq dequantized on the fly,
 * and fp32 accumulation.
 *
 * Sources, cited by page title and section (all are web pages about the ZSE
 * inference engine):
 *   [wiki]  the wiki.iphoster.net article "ZSE - open-source движок для запуска
 *           LLM локально на GPU - 2026"
 *   [ocr]   the openclawradar.com articles "ZSE: Motor de inferência de LLM de
 *           código aberto ..." (pt) and "ZSE: Open-Source-LLM-Inferenz-Engine
 *           ..." (de)
 *   [lavx]  the news.lavx.hu article "ZSE: A Memory-Efficient LLM Inference
 *           Engine with Smart Resource Orchestration"
 *
 * ---------------------------------------------------------------------------
 * Packed weight format (fixed by this library)
 *   [wiki, section "Формат модели .zse"] quantizes groups of 128 weights, packs
 *   two 4-bit values per byte with the low nibble first, keeps fp16 scales and
 *   quantizes at conversion time rather than at load time. [ocr, section
 *   "Componentes da arquitetura"; lavx, section "Technical Architecture"]
 *   describe zQuantize as per-tensor INT2..INT8 mixed precision. This library
 *   keeps the group size, the nibble order and the fp16 scales, and uses
 *   symmetric signed codes (no zero point):
 *   - bits b in {2, 4, 8}; codes q are two's complement in [-2^(b-1), 2^(b-1)-1];
 *   - codes run along K; 8/b codes per byte; code i of a byte sits in bits
 *     [b*i + b-1 : b*i] (INT4: even k in the low nibble); rows are dense,
 *     row r starts at byte r * k*b/8; no padding;
 *   - scales are IEEE binary16 bit patterns: group = 0 -> one scale for the
 *     whole tensor; group = 128 -> one per row and per 128 consecutive k,
 *     laid out [n][k/128] row-major;
 *   - w_deq[n][k] = q[n][k] * scale(n, k).
 *
 * Conventions for every call
 *   - Pointers named "device" are device memory owned by the caller (for
 *     example a torch tensor's data_ptr()). The library never frees or keeps
 *     them. zq_gemv / zq_gemm / zq_unpack allocate nothing.
 *   - `stream` is a hipStream_t (NULL = the null stream). gemv, gemm and
 *     unpack only enqueue work on it and return; faults inside a kernel
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Every argument is validated before any HIP call. A failed check returns
 *     ZQ_ERR_INVALID_ARG (null pointer, negative size, leading dimension too
 *     small, dtype not accepted by the call) or ZQ_ERR_UNSUPPORTED (bits not
 *     in {2,4,8}, group not in {0,128}, k not a multiple of the group or of
 *     8/bits); nothing is launched and nothing aborts. ZQ_ERR_HIP reports a
 *     failed HIP runtime call. zq_last_error() then holds a one-line detail
 *     for the calling thread.
 *   - Fast paths want 16-byte aligned pointers and rows whose byte length is a
 *     multiple of 16; any other legal shape runs on a slower general kernel
 *     with the same results.
 *   - Sizes are element counts (int64_t). n == 0, k == 0 or m == 0 is legal
 *     and does nothing (k == 0 with n > 0 writes zeros).
 * ---------------------------------------------------------------------------
 */
#ifndef ZQ_H
#define ZQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below have int as their underlying type, so that any int
 * a C caller passes is a valid value to validate (C enums are ints). */
#ifdef __cplusplus
#define ZQ_ENUM_BASE : int
#else
#define ZQ_ENUM_BASE
#endif

typedef enum ZQ_ENUM_BASE {
  ZQ_OK = 0,
  ZQ_ERR_INVALID_ARG = 1,
  ZQ_ERR_UNSUPPORTED = 2,
  ZQ_ERR_RANGE = 3,  /* non-finite input, scale beyond fp16, code out of range */
  ZQ_ERR_HIP = 4
} zq_status;

typedef enum ZQ_ENUM_BASE {
  ZQ_I8 = 0,   /* int8 integer codes */
  ZQ_F16 = 1,  /* IEEE binary16 */
  ZQ_BF16 = 2, /* bfloat16 */
  ZQ_F32 = 3   /* IEEE binary32 */
} zq_dtype;

/* A packed weight matrix resident in device memory (nn.Linear layout [n][k]). */
typedef struct zq_weight {
  int32_t bits;           /* 2, 4 or 8 */
  int32_t group;          /* 0: one scale per tensor; 128: per row and 128 k */
  int64_t n;              /* output features (rows) */
  int64_t k;              /* input features */
  const void* packed;     /* device, zq_packed_bytes(bits, n, k) bytes */
  const uint16_t* scales; /* device, zq_num_scales(group, n, k) fp16 patterns */
  const uint16_t* zeros;  /* NULL: symmetric signed codes (above). Non-NULL:
                           * asymmetric weights -- device, n * (k / 128) fp16
                           * zero points laid out like the scales; codes are
                           * unsigned in [0, 2^b - 1] and w_deq = q * s + z;
                           * bits 2 or 4 and group 128 only. */
} zq_weight;

/* Bytes of packed codes: n * k * bits / 8. Returns 0 for unsupported bits.
 * [wiki, section "Формат модели .zse": two INT4 values per byte; zQuantize
 * (openclawradar, section "Componentes da arquitetura") stores INT2 and INT8
 * tensors the same way, 4 and 1 codes per byte.] */
size_t zq_packed_bytes(int bits, int64_t n, int64_t k);

/* Number of fp16 scales: 1 for group 0, n * (k / 128) for group 128;
 * -1 for an unsupported group. [wiki, section "Формат модели .zse": one fp16
 * scale per group of 128 weights; zQuantize's per-tensor variant: one per
 * tensor.] */
int64_t zq_num_scales(int group, int64_t n, int64_t k);

/*
 * zq_pack -- quantize (when given floats) and pack one weight matrix.
 * [wiki, section "Формат модели .zse": quantization happens once, when a
 * model is converted; groups of 128; two INT4 per byte, low nibble first.]
 *
 *   w          device, [n][k] row-major, dtype w_dtype:
 *              ZQ_I8  -- ready-made integer codes: pure bit packing. Codes
 *                        outside [-2^(b-1), 2^(b-1)-1] give ZQ_ERR_RANGE.
 *                        scales_in, if non-NULL, is copied to scales_out.
 *              ZQ_F16 / ZQ_BF16 / ZQ_F32 -- float weights to quantize.
 *   scales_in  device, NULL or zq_num_scales fp16 patterns fixed by the
 *              caller. NULL with float weights: scales are computed per unit
 *              (the tensor, or 128 k of one row) as
 *                a = max|w|; a == 0 -> scale +0;
 *                else s = fp16_round_nearest_even(a / qmax), qmax = 2^(b-1)-1,
 *                raised to the next fp16 when s * qmax < a (so no code clips);
 *              given scales are used as they are and codes clip.
 *   codes      q = clamp(round_half_even(w / s), -2^(b-1), 2^(b-1)-1), the
 *              division in double; s == 0 gives q = 0.
 *   packed_out device, zq_packed_bytes(bits, n, k) bytes, written.
 *   scales_out device, zq_num_scales fp16 patterns, written (may be NULL only
 *              when w_dtype is ZQ_I8 or when scales_in is given).
 * Synchronous: returns after the work on `stream` has finished.
 * ZQ_ERR_RANGE for a non-finite weight or scale, or a scale beyond the fp16
 * range; packed_out / scales_out contents are then unspecified. It allocates
 * and frees a few bytes of device memory for the error flag.
 */
/*
 * zq_pack_asym -- quantize and pack one weight matrix as asymmetric codes,
 * the .zse format's own quantizer. [wiki, section "Формат модели .zse":
 * asymmetric INT4 with a scale and a zero point per group of 128 weights,
 * both stored as fp16; scale = (max - min) / 15, zero = min, codes clamped to
 * [0, 15]; two values per byte, low nibble first.] For b bits the divisor is
 * qmax = 2^b - 1 (b in {2, 4}); the group is always 128 along K.
 *   w          device, [n][k] row-major, dtype w_dtype:
 *              ZQ_I8  -- ready-made unsigned codes in [0, qmax] (ZQ_ERR_RANGE
 *                        otherwise): pure bit packing; scales_in and zeros_in
 *                        are required and copied to scales_out / zeros_out
 *                        when those are non-NULL.
 *              ZQ_F16 / ZQ_BF16 / ZQ_F32 -- float weights to quantize.
 *   scales_in, zeros_in  device, both NULL or both n * (k / 128) fp16
 *              patterns. NULL with float weights: per group,
 *                s = fp16_round_nearest_even((max - min) / qmax),
 *                z = fp16_round_nearest_even(min);
 *   codes      q = clamp(round_half_even((w - z) / s), 0, qmax) with the
 *              stored fp16 s and z, in double; s == 0 gives q = 0.
 *   packed_out device, zq_packed_bytes(bits, n, k) bytes, written.
 *   scales_out, zeros_out  device, n * (k / 128) fp16 patterns each, written.
 * Synchronous, like zq_pack. ZQ_ERR_RANGE for a non-finite weight, or a scale
 * or zero beyond the fp16 range. The result is used through a zq_weight whose
 * `zeros` points at the zero points.
 */
zq_status zq_pack_asym(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits,
                       const uint16_t* scales_in, const uint16_t* zeros_in, void* packed_out,
                       uint16_t* scales_out, uint16_t* zeros_out, void* stream);

zq_status zq_pack(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits,
                  int group, const uint16_t* scales_in, void* packed_out,
                  uint16_t* scales_out, void* stream);

/*
 * zq_pack_noalloc -- zq_pack for callers that cannot allocate device memory
 * (code running under stream capture elsewhere in the process, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments, results, errors
 * and synchronous behaviour as zq_pack, bit for bit; it calls no hipMalloc,
 * hipFree or other allocating routine.
 *   Scratch: the pack kernels' two flag words (error bits, tensor absmax) live
 *   in a 256-byte device array inside the library, one copy per GPU, held
 *   until the process ends; its address is looked up on the first call on
 *   each device. Every shape that zq_pack accepts fits it (the flags do not
 *   grow with n or k), so no size is rejected beyond zq_pack's own checks.
 *   The words are cleared at the start of every call.
 *   Calls that overlap on one GPU (other host threads or streams) share that
 *   array and race: serialise them.
 */
zq_status zq_pack_noalloc(const void* w, zq_dtype w_dtype, int64_t n, int64_t k, int bits,
                          int group, const uint16_t* scales_in, void* packed_out,
                          uint16_t* scales_out, void* stream);

/*
 * zq_unpack -- decode a packed matrix. [wiki, section "Компилятор GPU-ядер":
 * the unpack_int4 intrinsic; this is its signed form for 2, 4 and 8 bits.]
 *   out  device, [n][k] row-major of out_dtype:
 *        ZQ_I8  -- the integer codes, sign-extended (asymmetric weights: the
 *                  unsigned codes, 0 .. 2^b - 1);
 *        ZQ_F32 -- q * s exactly (asymmetric: q * s + z, rounded once);
 *        ZQ_F16 / ZQ_BF16 -- q * s (q * s + z) rounded to nearest even.
 * Asynchronous on `stream`.
 */
zq_status zq_unpack(const zq_weight* W, void* out, zq_dtype out_dtype, void* stream);

/*
 * zq_gemv -- decode step, one activation row: y[n] = sum_k x[k] * w_deq[n][k].
 * [wiki, section "Оркестратор и GPU-ядра": a hand-written wave-64 INT4 GEMV
 * with 128-bit weight loads is the main small-batch kernel on AMD; section
 * "Компилятор GPU-ядер": dequantizing matmuls are hand-written kernels.]
 *   W       packed weight (device pointers inside).
 *   x       device, k elements of x_dtype (ZQ_F16 or ZQ_BF16).
 *   y       device, n elements of y_dtype (ZQ_F32, ZQ_F16 or ZQ_BF16); the fp32
 *           sums are rounded to nearest even for F16 / BF16.
 * Asynchronous on `stream`. Same result as zq_gemm with m = 1.
 */
zq_status zq_gemv(const zq_weight* W, const void* x, zq_dtype x_dtype, void* y,
                  zq_dtype y_dtype, void* stream);

/*
 * zq_gemm -- batched decode and prefill: Y[m][n] = sum_k X[m][k] * w_deq[n][k].
 * [wiki, sections "Оркестратор и GPU-ядра" (small batches) and "Честные
 * ограничения" / "Перспективы" (concurrent INT4 decode at batch 4..16).]
 *   X       device, m rows of k elements, row stride ldx >= k elements,
 *           dtype ZQ_F16 or ZQ_BF16.
 *   Y       device, m rows of n elements, row stride ldy >= n, dtype ZQ_F32,
 *           ZQ_F16 or ZQ_BF16.
 * Kernels by shape (all give results within the same tolerance of the exact
 * sums; integer-valued inputs give exact sums on every path but one: the
 * group-scaled prefill tiles (m > 32) move their fp32 accumulators from one
 * group's scale to the next by a rounded ratio, exact only when the scales
 * of a row differ by powers of two, so there a one-hot row is a few ulp off
 * w_deq). Asymmetric
 * weights take the first three paths below, else the general kernel:
 *   m = 1, k a multiple of 128 (m <= 4 where the MFMA kernel below does
 *     not apply): a vector-ALU kernel that streams the codes once with
 *     128-bit loads;
 *   m = 2..32, INT4, k a multiple of 512, 16-byte aligned codes and
 *     activations, 8-byte aligned scales (and zero points): a resident MFMA
 *     kernel that streams the codes once;
 *   m > 32 (or 16 < m <= 32 in a format the kernel above does not take),
 *     symmetric codes, one scale per tensor (k a multiple of 64) or per row
 *     and 128 k, 16-byte aligned codes and activations: a tiled MFMA kernel
 *     (32, 64 or 128 x 256 tiles for m <= 32, <= 64 and above) that decodes
 *     codes in registers and applies group scales in fp32;
 *   asymmetric codes at m > 32, INT4, k a multiple of 512, aligned as
 *     above: the batched-decode kernel on chunks of 32 rows;
 *   anything else: tiled MFMA kernels, or a general kernel for unaligned and
 *     odd shapes.
 * Codes are decoded to bf16 / fp16 values that are exact for every code.
 * Asynchronous on `stream`.
 */
zq_status zq_gemm(const zq_weight* W, const void* X, zq_dtype x_dtype, int64_t m,
                  int64_t ldx, void* Y, zq_dtype y_dtype, int64_t ldy, void* stream);

/*
 * Plans: many decode-step products in one launch.
 * [wiki, section "Оркестратор и GPU-ядра": the decode launch sequence is
 * captured as one CUDA/HIP graph to cut launch cost.] On gfx950 a dependent
 * kernel launch costs more than streaming a small weight matrix, so a plan
 * runs a whole list of products in one resident launch instead.
 *
 * zq_problem   one product Y = X * dequant(W)^T, fields as in zq_gemm
 *              (m is the plan's). Problems run in array order of `phase`
 *              (non-decreasing in the array): every problem of phase p starts
 *              its arithmetic only after all problems of phases < p have
 *              stored their outputs, so Y of one phase may be X of the next
 *              (q,k,v -> o -> gate,up -> down of a decoder layer). Problems of
 *              one phase are independent and must not write what another one
 *              of that phase reads. The problems of a phase that share k,
 *              bits, group, zero points (present or not) and x dtype are
 *              streamed as one row space (any number of them, wherever they
 *              sit in the phase), split evenly over the workgroups.
 * zq_plan_create  validates every problem (as zq_gemm does) and requires
 *              m >= 1 (ZQ_ERR_UNSUPPORTED otherwise).
 *              m > 64 and every problem with symmetric codes, or 32 < m <=
 *              64 (16 < m <= 32 when some problem is not one the MFMA kernel
 *              below takes) and every problem one the prefill kernel takes,
 *              in one phase (prefill): one scale per tensor (k a multiple of 64) or
 *              per row and 128 k, 16-byte aligned codes and activations, one
 *              x dtype and one phase; the plan runs one persistent launch per
 *              bit width and scale kind present, whose workgroups take 32, 64
 *              or 128 x 256 output tiles from per-XCD device counters, so one
 *              run leaves no launch gaps between products and no idle CUs
 *              until its last round. Results are those of zq_gemm, bit for
 *              bit. Other plans with 32 < m: every problem INT4, k a multiple of 512,
 *              aligned as below; the rows run in chunks of 32 (never a last
 *              chunk of one row), each a plan of its own, so the weights
 *              stream once per chunk. For 2 <= m <= 32, when
 *              every problem is INT4 with k a multiple of 512, 16-byte aligned
 *              codes and activations and 8-byte aligned scales, the plan runs
 *              on the MFMA kernel; otherwise (m <= 4 only) on the vector-ALU
 *              kernel, which needs k a multiple of 128, 16-byte aligned
 *              pointers and activations of one problem
 *              that fit in the 160 KiB of LDS with their group sums (m * k * 2
 *              bytes plus 1/32 of that). The plan
 *              copies the list to device memory and allocates a few device
 *              words (phase or tile counters, error word, finished
 *              workgroups).
 *              Pointers inside the problems are used at every run: the caller
 *              keeps those buffers alive.
 * zq_plan_run  enqueues the plan on `stream`: one launch with one workgroup
 *              per CU (cooperative when the plan has more than one phase, so
 *              all workgroups are resident; prefill plans: one launch per
 *              bit width and scale kind, two to four workgroups per CU); allocates nothing; the run leaves
 *              the counter at zero for the next one. Runs of one plan that
 *              overlap (on different streams) race on its counter.
 * zq_plan_check synchronises the device and reports ZQ_ERR_HIP if a phase
 *              wait in an earlier run gave up (its outputs are then invalid).
 * zq_plan_destroy frees the plan's device memory (synchronises the device).
 */
typedef struct zq_problem {
  zq_weight w;
  const void* x;
  zq_dtype x_dtype;
  int64_t ldx;
  void* y;
  zq_dtype y_dtype;
  int64_t ldy;
  int32_t phase;
} zq_problem;

typedef struct zq_plan_s* zq_plan;

zq_status zq_plan_create(const zq_problem* problems, int count, int64_t m, zq_plan* plan_out);
zq_status zq_plan_run(zq_plan plan, void* stream);
zq_status zq_plan_check(zq_plan plan);
zq_status zq_plan_destroy(zq_plan plan);

/* Static description of a status code. The pages define no error
 * interface: the status codes and these two calls are this library's own
 * (the problem statement's calls -- zq_pack, zq_gemv, zq_gemm -- report
 * through them). */
const char* zq_status_string(zq_status s);

/* Detail of the last failed call made by this thread ("" if none); see
 * zq_status_string. */
const char* zq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ZQ_H */
