/*
 * moe_w2.h - C ABI of libmoew2.so: the routed Mixture-of-Experts expert forward over
 * sign-symmetric 2-bit weights, and the load-time NVFP4 -> 2-bit re-quantizer, for AMD MI355X
 * (gfx950).
 *
 * The method is the one described for vLLM-Moet ("The v0.24.0 port" page, section "Our hooks";
 * README bullets "2-bit expert planes - the sign-bias finding" and "The kernels"): routed expert
 * weights are 2-bit codes over the codebook {-4, -1, 1, 4} with one UE8M0 power-of-two scale per
 * 32 elements along each GEMM's reduction axis; the forward routes pairs (token, expert) to a
 * grouped gate/up GEMM, a SiLU-gated product, a grouped down GEMM and a router-weighted,
 * deterministic combine; NVFP4 experts (e2m1 x e4m3 block-16 x fp32 per-tensor scale_2) are
 * re-quantized to those planes at load time. Beside these: FP8 block-128 and MXFP4 re-quantizers,
 * FP4 (MXFP4) expert planes with the same forward, a slot-indexed forward for partially resident
 * experts, and the codebook sweep behind the sign-symmetric codebook choice.
 *
 * Conventions (all entry points):
 *  - Pointers are HIP device pointers unless a parameter says "host". The caller owns every
 *    buffer it passes and keeps it alive until the stream has passed the call. The library owns
 *    the native planes (moe_w2_planes), created by moe_w2_pack and freed by moe_w2_planes_free.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls are
 *    asynchronous on it unless marked "synchronous".
 *  - Every entry point returns a status (enum moe_w2_status). Host-detectable problems (null
 *    pointers, unsupported shapes, too small workspace) return a negative status before anything
 *    is enqueued. No call prints, aborts or throws.
 *  - Shapes: K (hidden size) and I (expert intermediate size) must be multiples of 256 with
 *    I*K < 2^32;
 *    1 <= E <= 1024; 1 <= top_k <= 32; T >= 0 (T = 0 is a no-op); T*top_k <= 2^30 in every
 *    entry point that takes T (moe_w2_workspace_bytes and moe_w2_route_workspace_bytes return 0
 *    above it, the others MOE_W2_EUNSUPPORTED). A forward also needs
 *    T*K < 2^31 and T*top_k*I < 2^31 (element counts of x and of the gated intermediate),
 *    T*(K/256)*608 < 2^32 and T*top_k*(I/256)*608 < 2^32 (bytes of their split copies).
 *
 * Canonical plane layout (the input of moe_w2_pack, the output of nvfp4_to_w2):
 *  - codes: 4 per byte along the row's reduction axis, element k at bits 2*(k%4)..+1 (LSB
 *    first); code c in 0..3 has value {-4, -1, +1, +4}[c] (code order from the starlog article,
 *    section "Technical Insight"; c and 3-c are negatives).
 *  - scales: one UE8M0 byte per 32 elements along the reduction axis: value 2^(b-127).
 *  - gate_up[e] has 2I rows of K: rows 0..I-1 are the gate projection, rows I..2I-1 the up
 *    projection. down[e] has K rows of I.
 */
#ifndef MOE_W2_H
#define MOE_W2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_w2_status {
  MOE_W2_OK = 0,
  MOE_W2_EINVAL = -1,        /* null pointer, negative size or bad enum value */
  MOE_W2_EUNSUPPORTED = -2,  /* shape outside the supported set (see conventions above) */
  MOE_W2_ESCALE = -3,        /* a scale byte outside the range the planes can hold */
  MOE_W2_ENOMEM = -4,        /* device allocation failed */
  MOE_W2_EHIP = -5,          /* a HIP runtime call failed */
  MOE_W2_EWORKSPACE = -6,    /* workspace null or smaller than moe_w2_workspace_bytes() */
  MOE_W2_ENVFP4 = -7,        /* NaN e4m3 byte or NaN / infinite scale_2 in nvfp4_to_w2 input */
  MOE_W2_ENAN = -8           /* NaN element or scale, or non-finite scale, in fp8_block128_to_w2 /
                                mxfp4_to_w2 input */
};

enum moe_w2_out_dtype { MOE_W2_OUT_BF16 = 0, MOE_W2_OUT_F32 = 1 };

/* Which kernels moe_w2_forward uses. AUTO picks the decode kernels for T*top_k <= 512, else
 * GEMM; among the decode organisations,
 * DECODE_SORTED from 384 pairs up, DECODE below. DECODE supports T*top_k <= 512 only
 * (MOE_W2_EUNSUPPORTED above); DECODE_SORTED any number of pairs P = T*top_k with
 * P/4 + min(E, P) + 1 <= 65535 (its launch has that many workgroup rows, one per chunk of up to 4
 * pairs of one expert). DECODE streams an expert's weights once per 4 of its pairs, finding
 * each expert's pairs from the ids inside the kernels (no routing pass). DECODE_SORTED runs a
 * routing pass first and walks its chunks in expert order, so the chunks of a popular expert run
 * together; up to 512 pairs it groups an expert's pairs by 16 and splits a group's reductions
 * over workgroups, so its weights stream once per 16 pairs. All paths give results within the
 * same tolerance; the two decode organisations give bit-identical results when no expert has
 * more than 4 pairs (same per-pair arithmetic), and otherwise differ only by the order of the
 * fp32 sums of a split reduction. */
enum moe_w2_path {
  MOE_W2_PATH_AUTO = 0,
  MOE_W2_PATH_DECODE = 1,
  MOE_W2_PATH_GEMM = 2,
  MOE_W2_PATH_DECODE_SORTED = 3
};

/* The four stages of moe_w2_forward, in order (see moe_w2_forward_stage). */
enum moe_w2_stage {
  MOE_W2_STAGE_ROUTE = 0,    /* token sort / expert offsets / tile lists, into the workspace */
  MOE_W2_STAGE_GATE_UP = 1,  /* grouped gate/up GEMM + SiLU-gated product -> workspace */
  MOE_W2_STAGE_DOWN = 2,     /* grouped down GEMM -> per-pair rows in the workspace */
  MOE_W2_STAGE_COMBINE = 3   /* router-weighted fixed-order combine -> y */
};

typedef struct moe_w2_planes moe_w2_planes; /* opaque; library-owned native planes */

/* ABI version of this header (increases on incompatible change). */
int moe_w2_abi_version(void);

/* Static description of a status code (never NULL). */
const char* moe_w2_status_string(int status);

/*
 * moe_w2_pack - build the native planes of one MoE layer from canonical planes.
 * Source: "The v0.24.0 port", section "Our hooks" (planes are built when weights are processed
 * after loading; four sections per expert: gate_up codes, gate_up scales, down codes, down
 * scales).
 *   gu_codes  [E][2I][K/4]   gu_scales [E][2I][K/32]
 *   dn_codes  [E][K][I/4]    dn_scales [E][K][I/32]
 * The native layout is opaque (tiles of 16 rows x 256 reduction elements in the operand order
 * of the block-scaled matrix instruction; gate and up rows interleaved in groups of 16). Every
 * scale byte must be <= 252 (a weight 4 * 2^(b-127) must be finite in fp32); MOE_W2_ESCALE
 * otherwise.
 * Synchronous (validates the scale bytes on the device). On success *out receives the planes;
 * on failure nothing is allocated and *out is NULL.
 */
int moe_w2_pack(int E, int K, int I,
                const uint8_t* gu_codes, const uint8_t* gu_scales,
                const uint8_t* dn_codes, const uint8_t* dn_scales,
                void* stream, moe_w2_planes** out);

/*
 * moe_w4_pack - native planes of one MoE layer with FP4 (MXFP4) experts: e2m1 codes with one
 * UE8M0 scale per 32 elements along each GEMM's reduction axis. Source: README bullet "FP4
 * recovery - used surgically" (a delta tier keeps hot experts at FP4; an FP4 read is twice the
 * bytes of the 2-bit planes) and bullet "The kernels" (the moe_w4_mm FP4 GEMM beside moe_w2_mm).
 *   gu_codes  [E][2I][K/2]  two e2m1 codes per byte, low nibble = even element
 *   gu_scales [E][2I][K/32] dn_codes [E][K][I/2] dn_scales [E][K][I/32]
 * e2m1 code n: sign n>>3, magnitude {0, 0.5, 1, 1.5, 2, 3, 4, 6}[n & 7]; weight = value * 2^(b-127).
 * Scale bytes must be <= 252 (MOE_W2_ESCALE otherwise); also needs I*K < 2^31. The planes work
 * with moe_w2_forward / moe_w2_forward_stage / moe_w4_forward (same arithmetic, fp4 weights in
 * place of the expanded 2-bit codes). Synchronous, like moe_w2_pack.
 */
int moe_w4_pack(int E, int K, int I,
                const uint8_t* gu_codes, const uint8_t* gu_scales,
                const uint8_t* dn_codes, const uint8_t* dn_scales,
                void* stream, moe_w2_planes** out);

/*
 * moe_w4_pack_nvfp4 - native planes of one MoE layer with NVFP4 experts: e2m1 codes, one
 * E4M3FN scale per 16 elements along each GEMM's reduction axis and one fp32 scale_2 per tensor,
 * weight = e2m1 x e4m3 x scale_2. Source: README opening paragraph and bullet "FP4 recovery - used
 * surgically" (the NVFP4 checkpoint's experts kept at FP4 as a delta tier); "The v0.24.0 port",
 * section "Our hooks", modelopt.py bullet (the NVFP4 format: e2m1 x e4m3 block-16 x per-tensor
 * scale_2).
 *   gu_codes  [E][2I][K/2]  two e2m1 codes per byte, low nibble = even element
 *   gu_scales [E][2I][K/16] E4M3FN bytes        gu_scale2 [E][2] fp32: gate rows, up rows
 *   dn_codes  [E][K][I/2]   dn_scales [E][K][I/16]   dn_scale2 [E] fp32
 * A NaN scale byte (0x7F, 0xFF) or a non-finite scale_2 returns MOE_W2_ENVFP4; also needs
 * I*K < 2^31. The planes work with moe_w4_forward / moe_w2_forward / moe_w2_forward_stage on both
 * kernel families and every path: the block-scaled matrix instruction takes only power-of-two
 * block scales, so the weights enter the 16 x 16 x 32 bf16 (gate/up, with bf16 x) and fp16 (down,
 * with the fp16 gated product) instructions, e2m1 x e4m3 formed exactly in registers and scale_2
 * applied to the fp32 results. Synchronous, like moe_w2_pack.
 */
int moe_w4_pack_nvfp4(int E, int K, int I,
                      const uint8_t* gu_codes, const uint8_t* gu_scales, const float* gu_scale2,
                      const uint8_t* dn_codes, const uint8_t* dn_scales, const float* dn_scale2,
                      void* stream, moe_w2_planes** out);

/* Inverse of moe_w4_pack_nvfp4 into canonical buffers of its shapes (asynchronous; exact).
 * MOE_W2_EINVAL for other planes. */
int moe_w4_unpack_nvfp4(const moe_w2_planes* planes,
                        uint8_t* gu_codes, uint8_t* gu_scales, float* gu_scale2,
                        uint8_t* dn_codes, uint8_t* dn_scales, float* dn_scale2, void* stream);

/* Inverse of moe_w2_pack into canonical buffers of its shapes (asynchronous; exact).
 * MOE_W2_EINVAL for planes made by moe_w4_pack. */
int moe_w2_unpack(const moe_w2_planes* planes,
                  uint8_t* gu_codes, uint8_t* gu_scales,
                  uint8_t* dn_codes, uint8_t* dn_scales, void* stream);

/* Inverse of moe_w4_pack into canonical FP4 buffers (asynchronous; exact). MOE_W2_EINVAL for
 * planes made by moe_w2_pack. */
int moe_w4_unpack(const moe_w2_planes* planes,
                  uint8_t* gu_codes, uint8_t* gu_scales,
                  uint8_t* dn_codes, uint8_t* dn_scales, void* stream);

/* Free the planes (synchronous: waits for the device). NULL is a no-op. */
void moe_w2_planes_free(moe_w2_planes* planes);

/* Shape and device footprint of the planes. Host outputs; any of them may be NULL. */
int moe_w2_planes_info(const moe_w2_planes* planes, int* E, int* K, int* I, size_t* bytes);

/*
 * Workspace needed by moe_w2_forward for T tokens and top_k experts per token, in bytes
 * (0 on bad arguments). The workspace also holds the two device counters of moe_w2_read_counters.
 */
size_t moe_w2_workspace_bytes(const moe_w2_planes* planes, int T, int top_k);

/*
 * moe_w2_route - the token-sort / expert-offset pass on its own.
 * Source: "The v0.24.0 port", section "Our hooks", bullet "Deterministic unpermute": valid
 * sorted ids form a permutation of token*top_k+j.
 *   topk_ids [T][top_k] int32.  offsets [E+1] int32: offsets[e] = number of valid pairs with an
 *   expert id < e.  perm [T*top_k] int32: the pair indices p = t*top_k + j sorted by expert id,
 *   ascending p within an expert (stable); pairs whose id is outside [0, E) follow, ascending.
 *   workspace: device scratch of moe_w2_route_workspace_bytes(E, T, top_k) bytes.
 */
size_t moe_w2_route_workspace_bytes(int E, int T, int top_k);
int moe_w2_route(int E, int T, int top_k, const int32_t* topk_ids,
                 int32_t* offsets, int32_t* perm,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_w2_forward - y = sum_j w[t,j] * D_e (silu(G_e x_t) * (U_e x_t)), e = topk_ids[t,j].
 * Source: the method statement (top-k routed grouped GEMM: gate/up projection, SiLU-gated
 * product, down projection, router-weighted combine); README bullet "The kernels"; "The v0.24.0
 * port", bullet "Deterministic unpermute" (bijective per-pair placement, fixed-order sum).
 *   x        [T][K] bf16 (row-major)
 *   topk_ids [T][top_k] int32; ids outside [0, E) contribute nothing and are counted
 *   topk_w   [T][top_k] fp32 router weights
 *   y        [T][K] bf16 (MOE_W2_OUT_BF16, round-to-nearest-even of the fp32 result) or fp32
 *   workspace: device memory of at least moe_w2_workspace_bytes(planes, T, top_k) bytes; it
 *   must not be shared by forwards that may run concurrently.
 * Arithmetic: both projections run on the block-scaled matrix instruction (fp4 weights, fp8 or
 * fp6 activations) with fp32 accumulation. The weights enter exactly (codes as e2m1 values +-1,
 * +-4 under their UE8M0 block scale). The gated product silu(g) * u is rounded to fp16; an
 * intermediate above the fp16 range becomes +-inf and is counted (act_overflow). Activations
 * enter as parts with power-of-two scales per 32-value block:
 *  - PATH_DECODE: x as two e4m3 parts, exact for every bf16 value within 2^-11 of its block's
 *    largest magnitude; the fp16 gated product as three e4m3 parts, exact within 2^-10;
 *  - PATH_GEMM: x and the fp16 gated product each as three e2m3 parts whose sum is within
 *    2^-13 of the block's largest magnitude of every value.
 * Combine in fp32 with j ascending. A pair's result does not depend on which other pairs share
 * the call, the order in which pairs are processed, or where its expert's planes sit; repeated
 * calls are bit-identical.
 * Asynchronous; no host synchronisation and no allocation.
 */
int moe_w2_forward(const moe_w2_planes* planes, int T, int top_k,
                   const void* x, const int32_t* topk_ids, const float* topk_w,
                   void* y, int out_dtype,
                   void* workspace, size_t workspace_bytes, int path, void* stream);

/*
 * moe_w2_forward_noalloc - moe_w2_forward without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The workspace is a library-owned device array of MOE_W2_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held until the process ends; its address is looked up on the first call on
 * each device. The call allocates nothing (no hipMalloc, no allocating library routine).
 *   Arguments as moe_w2_forward, minus workspace/workspace_bytes; the planes must be on the
 *   current device (MOE_W2_EINVAL otherwise).
 *   Limit: moe_w2_workspace_bytes(planes, T, top_k) <= MOE_W2_NOALLOC_SCRATCH_BYTES, else
 *   MOE_W2_EUNSUPPORTED before anything is enqueued (e.g. up to 64 tokens x top-8 at K = 6144,
 *   I = 2048, E = 256, whose workspace is about 52 MB).
 *   Every call on a GPU shares that GPU's array, which keeps the last call's contents: calls
 *   that may overlap on one GPU (concurrent streams, or host threads) race and must be
 *   serialised by the caller; moe_w2_read_counters cannot read this workspace.
 */
#define MOE_W2_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_w2_forward_noalloc(const moe_w2_planes* planes, int T, int top_k,
                           const void* x, const int32_t* topk_ids, const float* topk_w,
                           void* y, int out_dtype, int path, void* stream);

/* moe_w4_forward - moe_w2_forward on planes made by moe_w4_pack or moe_w4_pack_nvfp4
 * (MOE_W2_EINVAL for others). */
int moe_w4_forward(const moe_w2_planes* planes, int T, int top_k,
                   const void* x, const int32_t* topk_ids, const float* topk_w,
                   void* y, int out_dtype,
                   void* workspace, size_t workspace_bytes, int path, void* stream);

/*
 * moe_w2_forward_stage - one stage of moe_w2_forward, with the same arguments. Calling stages
 * ROUTE, GATE_UP, DOWN, COMBINE in this order on one stream with one workspace is exactly
 * moe_w2_forward; each stage reads what the previous ones left in the workspace. Lets a caller
 * place events or other work between the stages. Asynchronous; no allocation.
 */
int moe_w2_forward_stage(const moe_w2_planes* planes, int stage, int T, int top_k,
                         const void* x, const int32_t* topk_ids, const float* topk_w,
                         void* y, int out_dtype,
                         void* workspace, size_t workspace_bytes, int path, void* stream);

/*
 * Device counters of the last forward that used `workspace` (synchronous: waits for `stream`).
 * invalid_pairs: pairs whose id was outside [0, E). act_overflow: gated intermediates that
 * overflowed fp16. Host outputs.
 */
int moe_w2_read_counters(const void* workspace, int64_t* invalid_pairs, int64_t* act_overflow,
                         void* stream);

/*
 * Expert slots: planes of S slots, each holding one expert's planes, and a forward that reaches
 * experts through a device map expert -> slot. Source: the README paragraph on the base cache
 * (the GPU holds a cache of hot experts in the slot machinery; a missing expert's contribution
 * is zeroed and an in-graph miss counter bumped; after the missing experts are fetched the step
 * is replayed, bit-identical to a fully resident forward); "The v0.24.0 port", section "Our
 * hooks", BASE cache bullet (slot table, four sections per expert slot); "vLLM-Moet: a 2-bit
 * expert patch and a three-tier expert cache on SM120", section "A cache miss costs a replay".
 *
 * moe_w2_planes_create - planes of S empty 2-bit slots for K and I (contents unspecified until
 * packed).
 * Synchronous. On failure *out is NULL.
 */
int moe_w2_planes_create(int S, int K, int I, void* stream, moe_w2_planes** out);

/*
 * moe_w2_pack_slot - pack one expert's canonical planes into slot `slot` of `planes`:
 *   gu_codes [2I][K/4]  gu_scales [2I][K/32]  dn_codes [K][I/4]  dn_scales [K][I/32]
 * (the layout of one expert of moe_w2_pack). Synchronous (validates the scale bytes); on
 * MOE_W2_ESCALE the slot's contents are unspecified. Must not overlap a forward that reads the
 * slot.
 */
int moe_w2_pack_slot(moe_w2_planes* planes, int slot,
                     const uint8_t* gu_codes, const uint8_t* gu_scales,
                     const uint8_t* dn_codes, const uint8_t* dn_scales, void* stream);

/*
 * moe_w2_forward_slots - moe_w2_forward over experts 0..E-1 reached through slot_of_expert
 * [E] int32 (device): expert e's planes are in slot slot_of_expert[e] of `planes` (which has S
 * slots), or nowhere when the entry is outside [0, S). A pair whose expert is in no slot (a
 * miss) contributes nothing, like an id outside [0, E); both are counted in invalid_pairs, and
 * misses alone in the miss counter (moe_w2_read_miss_counter). Every pair whose expert is
 * resident gets exactly the result moe_w2_forward gives it on planes packed in expert order, so
 * once the missing experts are packed into slots and the map updated, the same call is
 * bit-identical to a fully resident forward. Workspace: moe_w2_workspace_bytes(planes, T, top_k).
 * Other arguments and behaviour as moe_w2_forward. Asynchronous; no allocation.
 */
int moe_w2_forward_slots(const moe_w2_planes* planes, int E, const int32_t* slot_of_expert,
                         int T, int top_k, const void* x, const int32_t* topk_ids,
                         const float* topk_w, void* y, int out_dtype,
                         void* workspace, size_t workspace_bytes, int path, void* stream);

/* Misses of the last moe_w2_forward_slots that used `workspace` (synchronous). Host output. */
int moe_w2_read_miss_counter(const void* workspace, int64_t* miss_pairs, void* stream);

/*
 * nvfp4_to_w2 - load-time re-quantizer NVFP4 -> canonical 2-bit planes.
 * Source: "The v0.24.0 port", section "Our hooks", modelopt.py bullet (exact f64 dequant of
 * e2m1 codes x f8e4m3 block-16 scales x per-tensor weight_scale_2; re-quantization to the
 * sign-symmetric codebook; UE8M0 block-32 output scales absorb scale_2); README opening
 * paragraph.
 *   e2m1    [n][R][C/2]  two e2m1 codes per byte, low nibble = even element
 *   e4m3    [n][R][C/16] E4M3FN block scales (one per 16 elements)
 *   scale_2 [n]          fp32 per-tensor scale
 *   codes   [n][R][C/4]  canonical codes;  scales [n][R][C/32] UE8M0 bytes
 * Per 32-element block: x = e2m1 * e4m3 * scale_2 (exact); the exponent e in [-127, 127] and
 * per-element magnitudes q in {1, 4} minimise sum (|x| - q 2^e)^2 exactly; equal errors take the
 * lower exponent; |x| exactly 2.5 * 2^e takes q = 1; the code sign is the sign bit of x (-0 is
 * negative). C must be a multiple of 32; n, R >= 0.
 * Synchronous; returns MOE_W2_ENVFP4 if any e4m3 byte is NaN (0x7F/0xFF) or a scale_2 is NaN or
 * infinite (outputs for the affected blocks are then unspecified).
 */
int nvfp4_to_w2(int n, int R, int C,
                const uint8_t* e2m1, const uint8_t* e4m3, const float* scale_2,
                uint8_t* codes, uint8_t* scales, void* stream);

/*
 * fp8_block128_to_w2 - load-time re-quantizer FP8 block-quant -> canonical 2-bit planes.
 * Source: "The v0.24.0 port", section "Our hooks", fp8.py bullet (FP8 block-quant checkpoints:
 * fp8 weights with fp32 block-128 scales re-quantized to the sign-symmetric codebook at load in
 * float64 math); README: the three checkpoint flavours that load.
 *   e4m3   [n][R][C]          E4M3FN weights
 *   bscale [n][R/128][C/128]  fp32 scale of each 128 x 128 block (reading: the usual block-quant
 *                             layout; the pages name "block-128" only)
 *   codes  [n][R][C/4], scales [n][R][C/32]  as nvfp4_to_w2
 * x = e4m3 * bscale (exact: 4 + 24 significant bits); then exactly nvfp4_to_w2's choice per
 * 32-element block (exponent minimising the exact squared error over [-127, 127], ties to the
 * lower exponent, |x| = 2.5 * 2^e -> magnitude 1, sign from the sign bit of x).
 * R and C multiples of 128. Synchronous; MOE_W2_ENAN for a NaN e4m3 byte or a non-finite scale
 * (the affected blocks' outputs are then unspecified).
 */
int fp8_block128_to_w2(int n, int R, int C, const uint8_t* e4m3, const float* bscale,
                       uint8_t* codes, uint8_t* scales, void* stream);

/*
 * mxfp4_to_w2 - load-time re-quantizer MXFP4 (e2m1 with UE8M0 block-32 scales, the FP4
 * checkpoints' experts; README: "FP4 experts ... codes remap") -> canonical 2-bit planes.
 *   e2m1 [n][R][C/2] (low nibble = even element), ue8m0 [n][R][C/32]; outputs as nvfp4_to_w2.
 * x = e2m1 * 2^(b-127) exactly, then nvfp4_to_w2's choice per block (reading: the "codes remap"
 * of the FP4 flavour is this exact re-quantization; an e2m1 code has 16 values, the 2-bit code 4,
 * so no plain remap exists). C a multiple of 32. Synchronous; MOE_W2_ENAN for a scale byte 255.
 */
int mxfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* ue8m0,
                uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_w2_codebook_sweep - sign-bias diagnostic of 2-bit codebooks. README, bullet "2-bit expert
 * planes - the sign-bias finding", and the vLLM-Moet article, section "Sign symmetry, not error
 * size, is what collapses naive 2-bit experts": the L2-optimal 2-bit codebook is sign-asymmetric
 * and leaves a per-tensor bias, the symmetric {-4,-1,1,4} reaches the same relative RMS error
 * with a far smaller bias; a codebook sweep over expert tensors measures both.
 *   x          [n][R][C] fp32, device, 16-byte aligned; blocks of 32 along C (C % 32 == 0)
 *   codebooks  [M][4] fp32, HOST, each strictly ascending and finite; 1 <= M <= 4096
 *   stats      [n][M][4] float64, device: {sse, err, rel_rms, bias} of tensor t under codebook m
 *   moments    [n][2] float64, device: {sum x^2, sum x}
 *   best       [n][2] int32, device: least-sse codebook with q0 = -q3 and q1 = -q2, and least-sse
 *              other codebook (ties to the lower index; -1 if there is none of that kind)
 * Quantization per codebook (readings where the pages are silent): scale 2^e per block, e in
 * [-127, 127] (the planes' UE8M0 block-32 scale); nearest code, halfway -> the code of smaller
 * magnitude, x = +-0 between q and -q -> the side of its sign bit; e minimises the block's
 * squared error over the ten exponents from 7 below to 2 above e_c, the least e with
 * max(|q0|,|q3|) 2^e >= max|x| (e_c = -127 for an all-zero block), equal errors to the lower e;
 * a block's squared error is summed in float64 in element order without fused operations.
 * sse = sum of (v - x)^2, err = sum of (v - x), rel_rms = sqrt(sse / sum x^2), bias =
 * err / sqrt(N sum x^2) (mean error over the rms of x; 0 when sum x^2 = 0), N = R * C.
 * Synchronous; allocates and frees its own scratch. MOE_W2_EINVAL for a bad codebook, pointer or
 * size, MOE_W2_EUNSUPPORTED for C % 32 != 0, MOE_W2_ENAN if x holds a NaN or an infinity (the
 * outputs are then unspecified).
 */
int moe_w2_codebook_sweep(int n, int R, int C, const float* x, int M, const float* codebooks,
                          double* stats, double* moments, int32_t* best, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W2_H */
