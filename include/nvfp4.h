/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 linear layer.
 *
 * The layer, as the pages describe it: activations and weights are NVFP4
 * tensors -- 4-bit E2M1 element codes, one E4M3 scale per 16-element block set
 * from the block maximum divided by 6, and one FP32 scale per tensor
 * (Summary page "Summary of 'Why Gated DeltaNet Survives 4-Bit Quantization'",
 * Background, item 1).  Activations are quantized on the fly at every call
 * ("W4A4", paper abstract).  Weights come from modules calibrated one by one,
 * each with its own FP32 scale; when several modules are fused into one GEMM,
 * each module's output columns must be rescaled with that module's own scale
 * -- the pages' repair of the global-scale mismatch (paper abstract; Glonce
 * article, "Who it affects" and "Risks and caveats"; aiany page,
 * "Mechanistic notes").  The segment table below is that per-module scale map.
 *
 * Conventions for every call:
 *  - Buffer pointers are DEVICE pointers unless marked "host".  The caller
 *    allocates and owns every buffer; the library never allocates, frees or
 *    retains device memory.  Its only global state is nvfp4_linear_noalloc's
 *    scratch: a static device array per GPU and the cached device addresses.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns without synchronizing;
 *    device-side faults surface at the caller's next synchronization.
 *    Kernels write into a call's workspace, so calls that share one must be
 *    ordered (one stream, or synchronized between streams).
 *  - Arguments are validated on the host before anything is launched: every
 *    status except NVFP4_EHIP means nothing was enqueued.  NVFP4_EHIP means the
 *    HIP runtime rejected a launch (hipGetLastError); a call that enqueues
 *    several kernels (the two-pass quantizer, nvfp4_linear outside its
 *    one-launch range, some GEMMs with a ragged last tile column) may already have
 *    enqueued the kernels before the rejected one, and all of its outputs are
 *    then unspecified.  The library never prints and never aborts.
 *  - Element codes are packed two per byte, the even k in the low nibble:
 *    byte j of a row = code[2j] | code[2j+1] << 4; code = sign << 3 | mag,
 *    mag 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Scales are E4M3FN bytes
 *    (0x00..0x7E).  Blocks of 16 run along K.
 *  - Every pointer must be 16-byte aligned, scalars and small tables included
 *    (NVFP4_EALIGN); K must be a multiple of 16.
 *  - Every row count, column count and leading dimension must be below 2^31
 *    (NVFP4_ESHAPE otherwise).
 */
#ifndef NVFP4_W4A4_H
#define NVFP4_W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: nvfp4_gemm_form may return 2 (the MFMA GEMM with 256 x 128 tiles). */
/* 3: nvfp4_read_probe. */
#define NVFP4_ABI_VERSION 3
#define NVFP4_MAX_SEGMENTS 16

typedef enum {
  NVFP4_OK = 0,
  NVFP4_EINVAL = 1,     /* null pointer, negative size, overlapping input/output buffers */
  NVFP4_ESHAPE = 2,     /* K % 16 != 0, leading dimension too small, a size or leading dimension >= 2^31 */
  NVFP4_EALIGN = 3,     /* pointer not 16-byte aligned, or bf16 leading dimension not a multiple of 8 */
  NVFP4_ESEGMENTS = 4,  /* segments do not tile [0, N) in order, or nseg not in [1, 16] */
  NVFP4_EWORKSPACE = 5, /* workspace missing or smaller than the *_workspace_bytes query */
  NVFP4_EHIP = 6        /* a kernel launch failed */
} nvfp4_status;

/* One fused module: output columns [n_begin, n_end) of the GEMM (rows of the weight). */
typedef struct {
  int32_t n_begin;
  int32_t n_end;
} nvfp4_segment;

/* Version of this ABI (NVFP4_ABI_VERSION).  Needs no GPU. */
int nvfp4_abi_version(void);

/* Static text for a status code.  Needs no GPU. */
const char* nvfp4_status_str(int status);

/* ---------------------------------------------------------------------------
 * Activation quantization (the "A4" of W4A4).
 *
 * Encodes bf16 activations x[M][K] (row stride ldx elements) to NVFP4 in the
 * canonical layout: codes[M][K/2] and scales[M][K/16], both row-major and
 * dense.  The per-tensor scale maps the tensor's absolute maximum amax onto
 * 6 * 448 = 2688 (the largest E2M1 magnitude times the largest E4M3 scale):
 *   g_enc = fl(2688 / amax), g_dec = fl(amax / 2688);
 *   per block: t = fl(bmax / 6), s = fl(t * g_enc), scale = E4M3(s)
 *              (round to nearest even, saturate at 448; t == 0 gives 0);
 *   per element: y = fl(|x| * fl(g_enc / s_dec)), mag = E2M1(y)
 *              (round to nearest even, saturate at 6; x == 0 or s_dec == 0
 *              gives 0); the sign bit is copied from x, -0.0 included.
 * amax == 0 gives g_dec = 0, scales 0 and sign-only codes.  Results are
 * bit-exact to that definition (binary32, no fused multiply-add).
 *
 *   amax_in   NULL: dynamic mode, amax = max|x| over the whole tensor.
 *             Otherwise a device pointer to one finite float >= 0 holding a
 *             calibrated amax (static mode); values of |x| above it saturate.
 *   g_dec_out device pointer to one float: receives g_dec.
 *   workspace device scratch of nvfp4_quantize_act_workspace_bytes(M, K)
 *             bytes (may be NULL when that is 0); contents need no setup.
 * Non-finite x are outside the contract (no fault; codes unspecified).
 * ------------------------------------------------------------------------- */
size_t nvfp4_quantize_act_workspace_bytes(int64_t M, int64_t K);

nvfp4_status nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, int64_t ldx,
                                const float* amax_in,
                                uint8_t* codes, uint8_t* scales, float* g_dec_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Weight packing (offline, post-training; the aiany page, "Who it's for",
 * describes the recipe as calibration-only post-training quantization).
 *
 * Encodes fp32 weights w[N][K] (row stride ldw elements) with the same rule
 * as the activations, module by module: each segment's rows get their own
 * amax and g_dec (w_g_dec[i], device, nseg floats).  Output is the tiled
 * weight layout the GEMM reads, with N padded to a multiple of 16 and K to a
 * multiple of 128 with zero codes and zero scales (sizes from
 * nvfp4_packed_weight_bytes).  The layout: chunks of 16 rows x 128 k, strip
 * major (chunk = (n / 16) * (Kp / 128) + k / 128), 1024 code bytes and 128
 * scale bytes per chunk.  Inside a chunk, the 16 canonical code bytes of row n,
 * k group g (k in [32 g, 32 g + 32)) sit at byte (16 g + n) * 16 and its two
 * scale bytes at byte (16 g + n) * 2, so lane l of a 64-lane wave reading bytes
 * [16 l, 16 l + 16) gets exactly the 16x16x32 MFMA operand of column l % 16,
 * k group l / 16.  `segs` is a HOST array.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_packed_weight_bytes(int64_t N, int64_t K, size_t* codes_bytes, size_t* scales_bytes);

size_t nvfp4_pack_weight_workspace_bytes(int64_t N, int64_t K, int32_t nseg);

nvfp4_status nvfp4_pack_weight(const float* w, int64_t N, int64_t K, int64_t ldw,
                               const nvfp4_segment* segs, int32_t nseg,
                               uint8_t* w_codes, uint8_t* w_scales, float* w_g_dec,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Unpack the tiled weight layout to canonical codes[N][K/2], scales[N][K/16]. */
nvfp4_status nvfp4_weight_to_canonical(const uint8_t* w_codes, const uint8_t* w_scales,
                                       int64_t N, int64_t K,
                                       uint8_t* codes, uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------
 * The W4A4 GEMM with the per-module global-scale epilogue.
 *
 *   out[m][n] = fl(acc[m][n] * fl(a_g_dec * w_g_dec[seg(n)]))
 *   acc[m][n] = sum_k (E2M1 * E4M3)(a)[m][k] * (E2M1 * E4M3)(w)[n][k]
 * with seg(n) the segment holding column n.  Every product is exact (the
 * operands are decoded exactly to fp16 and multiplied by the matrix cores);
 * the sum is accumulated in fp32 (FP32 accumulation; order unspecified).
 *
 *   a_codes/a_scales  canonical activations from nvfp4_quantize_act, M x K.
 *   a_g_dec           device pointer to the activations' g_dec.
 *   w_codes/w_scales  tiled weights from nvfp4_pack_weight, N x K.
 *   segs              HOST array of nseg segments tiling [0, N) in order.
 *   w_g_dec           device array of nseg per-module g_dec values.
 *   out               fp32 [M][ldo], ldo >= N; must not overlap any input.
 * M <= 16 runs the bandwidth-bound skinny path; larger M the MFMA path, except
 * where too few 256 x 256 tiles would run to fill the chip (e.g. M up to ~256 at
 * K = 5120, N = 12288), which streams the weight once per 32 or 64 rows.  The
 * MFMA path uses 256 x 128 tiles where 256 x 256 tiles would leave a partial
 * last round (nvfp4_gemm_form).  The MFMA
 * path addresses its operands with 32-bit byte offsets: for M > 16 the activation
 * codes (M * K / 2 bytes) and the packed weight codes must each be below 4 GiB,
 * else NVFP4_ESHAPE.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec,
                        int64_t M, int64_t K,
                        const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                        const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg,
                        float* out, int64_t ldo, void* stream);

/* Which kernel form nvfp4_gemm (and the GEMM step of nvfp4_linear) runs for an
 * M x K x N product: 0 = the weight-streaming skinny GEMM (32 or 64 rows per
 * weight pass when M > 16), 1 = the MFMA GEMM with 256 x 256 output tiles,
 * 2 = the MFMA GEMM with 256 x 128 tiles (taken where the wide tiles would leave
 * a partial last round of the chip's CUs); -1 for negative sizes.
 * Informational: every form meets the same tolerance, and the two MFMA forms
 * give bit-identical results. */
int nvfp4_gemm_form(int64_t M, int64_t K, int64_t N);

/* ---------------------------------------------------------------------------
 * The whole W4A4 linear layer in one call: on-the-fly activation quantization
 * (as nvfp4_quantize_act) followed by the GEMM with the per-module epilogue (as
 * nvfp4_gemm).  The activation codes, scales and g_dec are written to the
 * caller's buffers as well, in the canonical layout.  Results are bit-identical
 * to calling nvfp4_quantize_act then nvfp4_gemm.
 *
 * Decode-sized inputs (1 <= M <= 16 with K <= 5120, M <= 8 with K <= 10240,
 * M <= 4 with K <= 20480) run as ONE launch: every GEMM workgroup encodes the
 * (small) activation tensor itself while its weight loads are in flight, so no
 * workspace and no hand-over between workgroups is needed.
 * Other inputs run the quantizer and the GEMM kernels back to back on the
 * stream (the GEMM's 4 GiB operand limit for M > 16 applies).
 *
 *   workspace  device scratch of nvfp4_linear_workspace_bytes(M, K) bytes
 *              (NULL allowed when that is 0 or amax_in is given); contents
 *              need no setup.  In dynamic mode it is written, so it must not
 *              overlap any input or output (NVFP4_EINVAL).
 * K == 0 writes g_dec and zero outputs; M == 0 writes g_dec only.
 * ------------------------------------------------------------------------- */
size_t nvfp4_linear_workspace_bytes(int64_t M, int64_t K);

nvfp4_status nvfp4_linear(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                          uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec,
                          const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                          const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg,
                          float* out, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream);

/* nvfp4_linear for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same call and results, with the workspace replaced by the library's own
 * scratch, a file-scope device array of 4112 bytes per GPU (enough for the
 * quantizer's partial maxima at every M and K; a workspace need beyond it
 * would be NVFP4_EWORKSPACE), held until the process ends.  Its device address
 * is looked up on the first call for the stream's GPU (NVFP4_EHIP if that
 * lookup fails, with nothing enqueued); the call itself allocates nothing.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap in
 * time on one GPU (different streams, not ordered) race; calls on one stream
 * are ordered.  The scratch needs no clearing: each call writes what it reads. */
nvfp4_status nvfp4_linear_noalloc(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                  uint8_t* a_codes, uint8_t* a_scales, float* a_g_dec,
                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                  const nvfp4_segment* segs, const float* w_g_dec, int32_t nseg,
                                  float* out, int64_t ldo, void* stream);

/* ---------------------------------------------------------------------------
 * Fused gate+up projection with the SwiGLU -> NVFP4 epilogue.
 *
 * Every linear layer is W4A4 (paper abstract), so the down projection's input
 * h = silu(g) * u, formed from the gate (g) and up (u) projections of the MLP,
 * is quantized on the fly too (Glonce article, "How to use it").  With a
 * calibrated maximum of h (static mode; calibration-only PTQ, aiany page,
 * "Who it's for") that quantization can run in the gate+up GEMM's epilogue,
 * which then never writes the fp32 gate/up output:
 *
 *   g, u  = the two modules' outputs exactly as nvfp4_gemm computes them
 *           (gate and up keep their own FP32 scales: the per-module repair);
 *   h     = bf16(silu(g) * u), silu(z) = z / (1 + e^-z), evaluated in fp32
 *           (round to nearest even to bf16);
 *   codes, scales, g_dec = nvfp4_quantize_act(h, amax_in = amax_h).
 * The fused kernel is the MFMA GEMM with this epilogue.  Its result is
 * bit-identical to nvfp4_gemm (unfused packing), nvfp4_swiglu and
 * nvfp4_quantize_act run one after another whenever that nvfp4_gemm takes the
 * MFMA form (nvfp4_gemm_form(M, K, 2I) is 1 or 2); where nvfp4_gemm takes the
 * weight-streaming form (small M) the two sum in different fp32 orders, and g
 * and u agree within the GEMM tolerance instead.
 * ------------------------------------------------------------------------- */

/* Pack a gate+up weight pair for nvfp4_gemm_swiglu_quantize.  w is fp32
 * [2I][K] (row stride ldw): rows [0, I) the gate module, [I, 2I) the up module,
 * each encoded with its own maximum (w_g_dec[0] gate, w_g_dec[1] up, device).
 * The packed layout is the tiled one of nvfp4_pack_weight for 2I rows taken in
 * interleaved order (packed row n = module (n / 128) % 2, row (n / 256) * 128 +
 * n % 128); sizes from nvfp4_packed_weight_bytes(2I, K).  Requires I % 128 == 0
 * and K >= 16; workspace of nvfp4_pack_weight_workspace_bytes(2I, K, 2). */
nvfp4_status nvfp4_pack_weight_gate_up(const float* w, int64_t I, int64_t K, int64_t ldw,
                                       uint8_t* w_codes, uint8_t* w_scales, float* w_g_dec,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* h's NVFP4 codes [M][I/2], scales [M][I/16] (canonical layout) and g_dec
 * (amax_h / 2688) from activations a (as for nvfp4_gemm) and a weight from
 * nvfp4_pack_weight_gate_up.  amax_h: device pointer to the calibrated maximum
 * of |h| (finite, >= 0; larger |h| saturate).  Requires I % 128 == 0, K >= 16,
 * and activation codes and packed weight codes each below 4 GiB (NVFP4_ESHAPE). */
nvfp4_status nvfp4_gemm_swiglu_quantize(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_g_dec,
                                        int64_t M, int64_t K, const uint8_t* w_codes, const uint8_t* w_scales,
                                        int64_t I, const float* w_g_dec, const float* amax_h,
                                        uint8_t* h_codes, uint8_t* h_scales, float* h_g_dec, void* stream);

/* The unfused SwiGLU step: h_bf16[m][j] = bf16(silu(gu[m][j]) * gu[m][I + j])
 * for a gate+up output gu (fp32, row stride ldgu >= 2I; h row stride ldh >= I),
 * with the arithmetic of the fused epilogue. */
nvfp4_status nvfp4_swiglu(const float* gu, int64_t M, int64_t I, int64_t ldgu, void* h_bf16, int64_t ldh,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Static (calibrated) activation scales.
 *
 * The pages' recipe is calibration-only post-training quantization (aiany
 * page, "Who it's for"): an activation's per-tensor maximum may be observed
 * over calibration batches and then passed as amax_in (static mode).
 *
 * nvfp4_amax_observe: *running_amax = max(*running_amax, max |x|) over the
 * bf16 tensor x[M][K] (row stride ldx); running_amax is a device float the
 * caller initializes (e.g. to 0).  Workspace: nvfp4_amax_observe_workspace_bytes.
 *
 * nvfp4_quantize_stats: with the static maximum *amax_in, counts (device
 * uint32[2], overwritten) receive the number of blocks whose unrounded scale
 * fl(fl(bmax / 6) * g_enc) exceeds 448 (the E4M3 encode saturates) and the
 * number of elements with y = fl(|x| * fl(g_enc / s_dec)) >= 7 (cut to the
 * largest E2M1 magnitude 6 rather than rounded to it: in saturated blocks or
 * under E4M3 subnormal scales), in the encoder's own binary32 steps.
 * amax == 0 counts nothing.
 * ------------------------------------------------------------------------- */
size_t nvfp4_amax_observe_workspace_bytes(int64_t M, int64_t K);

nvfp4_status nvfp4_amax_observe(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, float* running_amax,
                                void* workspace, size_t workspace_bytes, void* stream);

nvfp4_status nvfp4_quantize_stats(const void* x_bf16, int64_t M, int64_t K, int64_t ldx, const float* amax_in,
                                  uint32_t* counts, void* stream);

/* ---------------------------------------------------------------------------
 * Calibrated FP8 (E4M3FN) KV-cache codec, one scale per tensor.
 *
 * The quantized model is served with an FP8 KV cache under calibrated
 * per-tensor scales (paper abstract; Glonce article, "How to use it"; aiany
 * page, "Mechanistic notes").  Reading, built like the NVFP4 per-tensor scale:
 *   g_enc = fl(448 / amax), g_dec = fl(amax / 448)   (amax == 0: g = 0);
 *   code  = sign(x) << 7 | E4M3 RNE of fl(|x| * g_enc), saturating at 448;
 *   decode = bf16 (RNE) of fl(E4M3(code) * g_dec).
 * n elements, contiguous; amax is a device pointer to the calibrated maximum
 * (finite, >= 0).  Pointers 16-byte aligned; any n below 2^48 (NVFP4_ESHAPE
 * otherwise).  Non-finite x are outside the contract.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_kv_fp8_encode(const void* x_bf16, int64_t n, const float* amax, uint8_t* codes, void* stream);

nvfp4_status nvfp4_kv_fp8_decode(const uint8_t* codes, int64_t n, const float* amax, void* out_bf16, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostic: the device conversion steps the encoders and GEMMs are built
 * on, applied to the binary32 values with bit patterns first_bits + i,
 * i < n, so that tests can compare them with the format definitions over
 * whole ranges (e.g. every binary32 in [0, 8] or [0, 448]).  Values 2j and
 * 2j + 1 are converted as one pair, as the encoders pair elements.
 *   op 0  out[i] = E2M1 code (sign << 3 | magnitude code; nearest, ties to
 *         even, saturating at 6): the element step of every NVFP4 encoder.
 *   op 1  out[i] = E4M3FN code (nearest, ties to even, saturating at 448):
 *         the block-scale step and the FP8 KV-cache encode.
 *   op 2  out[2i], out[2i + 1] = fp16 bits (little endian) of the exact
 *         decode the GEMMs feed the matrix cores: E2M1 code (first_bits + i) & 15
 *         times E4M3 code ((first_bits + i) >> 4) & 127.
 * out holds n bytes (op 0, 1) or 2n bytes (op 2); first_bits + n <= 2^32
 * (NVFP4_ESHAPE otherwise); op outside 0..2 is NVFP4_EINVAL.
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_convert_sweep(int32_t op, uint32_t first_bits, int64_t n, uint8_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostic: the HBM read rate a stream of `bytes` reaches with the access
 * pattern of the decode-form GEMMs' weight stream -- the ceiling those GEMMs
 * are measured against.  `workgroups` workgroups of 512 lanes each read one
 * contiguous share of buf with non-temporal 16-byte loads (four in flight per
 * lane); workgroup b stores the XOR of every 32-bit word of its share to
 * sink[b], so that nothing is skipped and tests can check the coverage.
 *   buf   device, `bytes` bytes (a multiple of 16, below 2^40), read only.
 *   sink  device, `workgroups` uint32 words (1 <= workgroups <= 65536),
 *         disjoint from buf.
 * Pointers 16-byte aligned.  Errors as for every call (nothing enqueued unless
 * NVFP4_OK or NVFP4_EHIP).
 * ------------------------------------------------------------------------- */
nvfp4_status nvfp4_read_probe(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_W4A4_H */
