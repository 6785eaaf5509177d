// C ABI of libmoew2 (declared in include/moe_w2.h): argument checks, workspace layout and the
// sequence of kernel launches for each entry point.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "internal.h"

namespace moew2 {

Workspace workspace_layout(int E, int K, int I, int T, int top_k) {
  Workspace w;
  memset(&w, 0, sizeof(w));
  const int P = T * top_k;
  w.P = P;
  w.max_tiles = P > 0 ? P / kGemmBM + (E < P ? E : P) + 1 : 0;
  w.max_chunks = P > 0 ? P / kDecodeChunk + (E < P ? E : P) + 1 : 0;
  size_t o = 0;
  w.counters = o;  o += align_up(3 * sizeof(long long));
  w.offsets = o;   o += align_up((size_t)(E + 1) * 4);
  w.perm = o;      o += align_up((size_t)P * 4);
  w.active = o;    o += align_up((size_t)E * 4);
  w.meta = o;      o += align_up(8 * 4);
  w.tiles = o;     o += align_up((size_t)w.max_chunks * 2 * 4);   // max_chunks >= max_tiles
  const size_t rs = route_scratch_bytes(E, P);
  w.chunk_cnt = o;
  w.rank = o + (rs - align_up((size_t)P * 4));
  o += rs;
  w.xq = o;        o += align_up((size_t)T * (K / kTileK) * kA6Bytes);
  w.act = o;       o += align_up((size_t)P * I * 2);
  w.aq = o;        o += align_up((size_t)P * (I / kTileK) * kA6Bytes);
  w.pair_out = o;  o += align_up((size_t)P * K * 4);
  w.gu_part = o;   o += P <= kWideMaxPairs ? align_up((size_t)P * std::max(kWideSlices * 2 * I, K) * 4) : 0;
  w.pair_ncs = o;  o += align_up((size_t)P * 4);
  w.slot_ids = o;  o += align_up((size_t)P * 4);
  w.total = o;
  return w;
}

// The decode kernels address one expert's gate_up plane (2I x K codes, 2 bits each) as a buffer of
// at most 2^31 - 1 bytes.
static bool shape_ok(int E, int K, int I) {
  return E >= 1 && E <= 1024 && K >= 256 && I >= 256 && K % 256 == 0 && I % 256 == 0 &&
         (long long)I * K / 2 < (1LL << 31);
}

// Pair counts above 2^30 are not supported by any entry point (the kernels index pairs in 32 bits).
static bool pairs_ok(int T, int top_k) { return (long long)T * top_k <= (1LL << 30); }

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_W2_OK : MOE_W2_EHIP; }

// One device allocation holding E experts' (or slots') native planes and the validation flag.
static int planes_alloc(int E, int K, int I, int fmt, moe_w2_planes** out) {
  const size_t n_gu = (size_t)E * 2 * I * K;
  const size_t n_dn = (size_t)E * K * I;
  const int cb = code_bits(fmt), sg = scale_group(fmt);
  size_t o = 0;
  const size_t o_guc = o; o += align_up(n_gu * cb / 8);
  const size_t o_gus = o; o += align_up(n_gu / sg);
  const size_t o_dnc = o; o += align_up(n_dn * cb / 8);
  const size_t o_dns = o; o += align_up(n_dn / sg);
  const size_t o_s2 = o;  o += align_up((size_t)E * 3 * sizeof(float));
  const size_t o_flag = o; o += align_up(4);
  moe_w2_planes* p = new (std::nothrow) moe_w2_planes;
  if (!p) return MOE_W2_ENOMEM;
  memset(p, 0, sizeof(*p));
  p->E = E; p->K = K; p->I = I; p->fmt = fmt;
  if (hipGetDevice(&p->device) != hipSuccess) { delete p; return MOE_W2_EHIP; }
  if (hipMalloc(&p->base, o) != hipSuccess) { (void)hipGetLastError(); delete p; return MOE_W2_ENOMEM; }
  p->bytes = o;
  uint8_t* b = (uint8_t*)p->base;
  p->gu_codes = b + o_guc; p->gu_scales = b + o_gus;
  p->dn_codes = b + o_dnc; p->dn_scales = b + o_dns;
  p->scale2 = (float*)(b + o_s2);
  p->flag = (int32_t*)(b + o_flag);
  *out = p;
  return MOE_W2_OK;
}

// Reads the pack validation flag (synchronous).
static int pack_status(const moe_w2_planes* p, hipError_t err, hipStream_t s) {
  int32_t flag = 0;
  if (err == hipSuccess) err = hipMemcpyAsync(&flag, p->flag, 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return MOE_W2_EHIP;
  if (flag & kFlagNaN) return MOE_W2_ENVFP4;
  return (flag & kFlagScale) ? MOE_W2_ESCALE : MOE_W2_OK;
}

// Host-side checks shared by every forward entry point (nothing is enqueued).
static int forward_check(const moe_w2_planes* p, int T, int top_k, const void* x, const int32_t* topk_ids,
                         const float* topk_w, const void* y, int out_dtype, const void* workspace,
                         size_t workspace_bytes, int path) {
  if (!p || T < 0 || top_k < 1) return MOE_W2_EINVAL;
  if (top_k > 32) return MOE_W2_EUNSUPPORTED;
  if (out_dtype != MOE_W2_OUT_BF16 && out_dtype != MOE_W2_OUT_F32) return MOE_W2_EINVAL;
  if (path != MOE_W2_PATH_AUTO && path != MOE_W2_PATH_DECODE && path != MOE_W2_PATH_GEMM &&
      path != MOE_W2_PATH_DECODE_SORTED)
    return MOE_W2_EINVAL;
  if (T > 0 && (!x || !topk_ids || !topk_w || !y)) return MOE_W2_EINVAL;
  if (!pairs_ok(T, top_k)) return MOE_W2_EUNSUPPORTED;
  if ((long long)T * p->K >= (1LL << 31) || (long long)T * top_k * p->I >= (1LL << 31))
    return MOE_W2_EUNSUPPORTED;  // the GEMM kernels index x and the intermediate in 32 bits
  if ((long long)T * (p->K / kTileK) * kA6Bytes >= (1LL << 32) ||
      (long long)T * top_k * (p->I / kTileK) * kA6Bytes >= (1LL << 32))
    return MOE_W2_EUNSUPPORTED;  // ... and their split copies with 32-bit byte offsets
  const Workspace ws = workspace_layout(p->E, p->K, p->I, T, top_k);
  if (!workspace || workspace_bytes < ws.total) return MOE_W2_EWORKSPACE;
  // every decode workgroup of the routed organisation scans all ids itself (two per thread)
  if (path == MOE_W2_PATH_DECODE && (long long)T * top_k > kDecodeMaxPairs) return MOE_W2_EUNSUPPORTED;
  // the sorted organisation launches one workgroup row per chunk (grid rows are 16-bit)
  if (ws.max_chunks > 65535 && path == MOE_W2_PATH_DECODE_SORTED) return MOE_W2_EUNSUPPORTED;
  return MOE_W2_OK;
}

// Kernel family of a forward: -1 = grouped GEMMs, else the decode organisation.
static int decode_mode(int path, int P) {
  if (path == MOE_W2_PATH_GEMM || (path == MOE_W2_PATH_AUTO && P > kDecodeMaxPairs)) return -1;
  if (path == MOE_W2_PATH_DECODE_SORTED) return kDecodeSorted;
  if (P <= kDirectMaxPairs) return kDecodeDirect;
  if (path == MOE_W2_PATH_AUTO && P >= kSortedMinPairs) return kDecodeSorted;
  return kDecodeRouted;
}
}  // namespace moew2

using namespace moew2;

extern "C" {

int moe_w2_abi_version(void) { return 1; }

const char* moe_w2_status_string(int status) {
  switch (status) {
    case MOE_W2_OK: return "ok";
    case MOE_W2_EINVAL: return "invalid argument (null pointer, negative size or bad enum value)";
    case MOE_W2_EUNSUPPORTED: return "unsupported shape";
    case MOE_W2_ESCALE: return "scale byte out of the representable range";
    case MOE_W2_ENOMEM: return "device allocation failed";
    case MOE_W2_EHIP: return "HIP runtime error";
    case MOE_W2_EWORKSPACE: return "workspace missing or too small";
    case MOE_W2_ENVFP4: return "NaN e4m3 scale or non-finite scale_2 in NVFP4 input";
    case MOE_W2_ENAN: return "NaN element or scale, or non-finite scale, in FP8 / MXFP4 input";
    default: return "unknown status";
  }
}

static int pack_fmt(int fmt, int E, int K, int I, const uint8_t* gu_codes, const uint8_t* gu_scales,
                    const uint8_t* dn_codes, const uint8_t* dn_scales, void* stream, moe_w2_planes** out) {
  if (!out) return MOE_W2_EINVAL;
  *out = nullptr;
  if (!gu_codes || !gu_scales || !dn_codes || !dn_scales) return MOE_W2_EINVAL;
  if (E < 0 || K < 0 || I < 0) return MOE_W2_EINVAL;
  if (!shape_ok(E, K, I)) return MOE_W2_EUNSUPPORTED;
  // the decode kernels address one expert's gate_up codes as a buffer of at most 2^31 - 1 bytes
  if (fmt == kFmtW4 && (long long)I * K >= (1LL << 31)) return MOE_W2_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  moe_w2_planes* p = nullptr;
  int st = planes_alloc(E, K, I, fmt, &p);
  if (st != MOE_W2_OK) return st;
  st = pack_status(p, launch_pack(p, gu_codes, gu_scales, dn_codes, dn_scales, s), s);
  if (st != MOE_W2_OK) { (void)hipFree(p->base); delete p; return st; }
  *out = p;
  return MOE_W2_OK;
}

int moe_w2_pack(int E, int K, int I, const uint8_t* gu_codes, const uint8_t* gu_scales,
                const uint8_t* dn_codes, const uint8_t* dn_scales, void* stream,
                moe_w2_planes** out) {
  return pack_fmt(kFmtW2, E, K, I, gu_codes, gu_scales, dn_codes, dn_scales, stream, out);
}

int moe_w4_pack(int E, int K, int I, const uint8_t* gu_codes, const uint8_t* gu_scales,
                const uint8_t* dn_codes, const uint8_t* dn_scales, void* stream,
                moe_w2_planes** out) {
  return pack_fmt(kFmtW4, E, K, I, gu_codes, gu_scales, dn_codes, dn_scales, stream, out);
}

int moe_w4_pack_nvfp4(int E, int K, int I, const uint8_t* gu_codes, const uint8_t* gu_scales, const float* gu_scale2,
                      const uint8_t* dn_codes, const uint8_t* dn_scales, const float* dn_scale2, void* stream,
                      moe_w2_planes** out) {
  if (!out) return MOE_W2_EINVAL;
  *out = nullptr;
  if (!gu_codes || !gu_scales || !gu_scale2 || !dn_codes || !dn_scales || !dn_scale2) return MOE_W2_EINVAL;
  if (E < 0 || K < 0 || I < 0) return MOE_W2_EINVAL;
  if (!shape_ok(E, K, I) || (long long)I * K >= (1LL << 31)) return MOE_W2_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  moe_w2_planes* p = nullptr;
  int st = planes_alloc(E, K, I, kFmtNV4, &p);
  if (st != MOE_W2_OK) return st;
  st = pack_status(p, launch_pack_nv4(p, gu_codes, gu_scales, gu_scale2, dn_codes, dn_scales, dn_scale2, 0, s), s);
  if (st != MOE_W2_OK) { (void)hipFree(p->base); delete p; return st; }
  *out = p;
  return MOE_W2_OK;
}

int moe_w4_unpack_nvfp4(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales, float* gu_scale2,
                        uint8_t* dn_codes, uint8_t* dn_scales, float* dn_scale2, void* stream) {
  if (!p || !gu_codes || !gu_scales || !gu_scale2 || !dn_codes || !dn_scales || !dn_scale2) return MOE_W2_EINVAL;
  if (p->fmt != kFmtNV4) return MOE_W2_EINVAL;
  return hip_status(launch_pack_nv4(p, gu_codes, gu_scales, gu_scale2, dn_codes, dn_scales, dn_scale2, 1,
                                    (hipStream_t)stream));
}

int moe_w2_planes_create(int S, int K, int I, void* stream, moe_w2_planes** out) {
  (void)stream;
  if (!out) return MOE_W2_EINVAL;
  *out = nullptr;
  if (S < 0 || K < 0 || I < 0) return MOE_W2_EINVAL;
  if (!shape_ok(S, K, I)) return MOE_W2_EUNSUPPORTED;
  return planes_alloc(S, K, I, kFmtW2, out);
}

int moe_w2_pack_slot(moe_w2_planes* p, int slot, const uint8_t* gu_codes, const uint8_t* gu_scales,
                     const uint8_t* dn_codes, const uint8_t* dn_scales, void* stream) {
  if (!p || !gu_codes || !gu_scales || !dn_codes || !dn_scales) return MOE_W2_EINVAL;
  if (slot < 0 || slot >= p->E) return MOE_W2_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  return pack_status(p, launch_pack_experts(p, slot, 1, gu_codes, gu_scales, dn_codes, dn_scales, s), s);
}

int moe_w2_unpack(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales,
                  uint8_t* dn_codes, uint8_t* dn_scales, void* stream) {
  if (!p || !gu_codes || !gu_scales || !dn_codes || !dn_scales) return MOE_W2_EINVAL;
  if (p->fmt != kFmtW2) return MOE_W2_EINVAL;
  return hip_status(launch_unpack(p, gu_codes, gu_scales, dn_codes, dn_scales, (hipStream_t)stream));
}

int moe_w4_unpack(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales,
                  uint8_t* dn_codes, uint8_t* dn_scales, void* stream) {
  if (!p || !gu_codes || !gu_scales || !dn_codes || !dn_scales) return MOE_W2_EINVAL;
  if (p->fmt != kFmtW4) return MOE_W2_EINVAL;
  return hip_status(launch_unpack(p, gu_codes, gu_scales, dn_codes, dn_scales, (hipStream_t)stream));
}

void moe_w2_planes_free(moe_w2_planes* p) {
  if (!p) return;
  (void)hipDeviceSynchronize();
  (void)hipFree(p->base);
  delete p;
}

int moe_w2_planes_info(const moe_w2_planes* p, int* E, int* K, int* I, size_t* bytes) {
  if (!p) return MOE_W2_EINVAL;
  if (E) *E = p->E;
  if (K) *K = p->K;
  if (I) *I = p->I;
  if (bytes) *bytes = p->bytes;
  return MOE_W2_OK;
}

size_t moe_w2_workspace_bytes(const moe_w2_planes* p, int T, int top_k) {
  if (!p || T < 0 || top_k < 1 || top_k > 32 || !pairs_ok(T, top_k)) return 0;
  return workspace_layout(p->E, p->K, p->I, T, top_k).total;
}

size_t moe_w2_route_workspace_bytes(int E, int T, int top_k) {
  if (E < 1 || E > 1024 || T < 0 || top_k < 1 || top_k > 32 || !pairs_ok(T, top_k)) return 0;
  const int P = T * top_k;
  const int max_tiles = P / kGemmBM + (E < P ? E : P) + 1;
  return align_up((size_t)E * 4) + align_up(8 * 4) + align_up((size_t)max_tiles * 2 * 4) +
         route_scratch_bytes(E, P);
}

int moe_w2_route(int E, int T, int top_k, const int32_t* topk_ids, int32_t* offsets, int32_t* perm,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (E < 1 || T < 0 || top_k < 1) return MOE_W2_EINVAL;
  if (E > 1024 || top_k > 32 || !pairs_ok(T, top_k)) return MOE_W2_EUNSUPPORTED;
  if (!offsets || (T > 0 && (!topk_ids || !perm))) return MOE_W2_EINVAL;
  const size_t need = moe_w2_route_workspace_bytes(E, T, top_k);
  if (!workspace || workspace_bytes < need) return MOE_W2_EWORKSPACE;
  const int P = T * top_k;
  const int max_tiles = P / kGemmBM + (E < P ? E : P) + 1;
  uint8_t* w = (uint8_t*)workspace;
  RouteOut o;
  o.offsets = offsets;
  o.perm = perm;
  o.active = (int32_t*)w;  w += align_up((size_t)E * 4);
  o.meta = (int32_t*)w;    w += align_up(8 * 4);
  o.tiles = (int32_t*)w;   w += align_up((size_t)max_tiles * 2 * 4);
  o.chunk_cnt = (int32_t*)w;
  o.rank = (int32_t*)(w + route_scratch_bytes(E, P) - align_up((size_t)P * 4));
  o.counters = nullptr;
  o.max_tiles = max_tiles;
  o.tile_rows = kGemmBM;
  return hip_status(launch_route(E, T, top_k, topk_ids, o, (hipStream_t)stream));
}

int moe_w2_forward_stage(const moe_w2_planes* p, int stage, int T, int top_k, const void* x,
                         const int32_t* topk_ids, const float* topk_w, void* y, int out_dtype,
                         void* workspace, size_t workspace_bytes, int path, void* stream) {
  if (stage < MOE_W2_STAGE_ROUTE || stage > MOE_W2_STAGE_COMBINE) return MOE_W2_EINVAL;
  const int st = forward_check(p, T, top_k, x, topk_ids, topk_w, y, out_dtype, workspace, workspace_bytes, path);
  if (st != MOE_W2_OK) return st;
  const Workspace ws = workspace_layout(p->E, p->K, p->I, T, top_k);
  if (T == 0) return MOE_W2_OK;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* wsb = (uint8_t*)workspace;
  const int mode = decode_mode(path, T * top_k);
  const bool decode = mode >= 0;
  // the routed and direct decode organisations find their pairs from the ids themselves (no
  // routing pass); the direct organisation also combines inside the down stage
  const bool direct = mode == kDecodeDirect;
  hipError_t err = hipSuccess;
  switch (stage) {
    case MOE_W2_STAGE_ROUTE: {
      if (mode == kDecodeRouted || mode == kDecodeDirect) break;
      RouteOut o;
      o.offsets = (int32_t*)(wsb + ws.offsets);
      o.perm = (int32_t*)(wsb + ws.perm);
      o.active = (int32_t*)(wsb + ws.active);
      o.meta = (int32_t*)(wsb + ws.meta);
      o.tiles = (int32_t*)(wsb + ws.tiles);
      o.counters = (long long*)(wsb + ws.counters);
      o.chunk_cnt = (int32_t*)(wsb + ws.chunk_cnt);
      o.rank = (int32_t*)(wsb + ws.rank);
      o.max_tiles = mode == kDecodeSorted ? ws.max_chunks : ws.max_tiles;
      o.tile_rows = mode == kDecodeSorted ? kDecodeChunk : kGemmBM;
      o.wide = mode == kDecodeSorted && T * top_k <= kWideMaxPairs;
      err = launch_route(p->E, T, top_k, topk_ids, o, s);
      break;
    }
    case MOE_W2_STAGE_GATE_UP:
      err = decode ? launch_decode_gate_up(p, T, top_k, x, topk_ids, ws, wsb, mode, s)
                   : launch_gemm_gate_up(p, T, top_k, x, ws, wsb, s);
      break;
    case MOE_W2_STAGE_DOWN:
      err = decode ? launch_decode_down(p, T, top_k, topk_ids, topk_w, y, out_dtype, ws, wsb, mode, s)
                   : launch_gemm_down(p, T, top_k, ws, wsb, s);
      break;
    default:
      // the direct decode down stage already combined into y
      if (!direct) {
        // the sorted organisation's wide list splits the down stage of large groups in two halves
        const bool wide = mode == kDecodeSorted && T * top_k <= kWideMaxPairs;
        err = launch_combine(T, top_k, p->E, p->K, topk_ids, topk_w, (const float*)(wsb + ws.pair_out), y,
                             out_dtype, s, wide ? (const int32_t*)(wsb + ws.pair_ncs) : nullptr,
                             wide ? (const float*)(wsb + ws.gu_part) : nullptr);
      }
  }
  return hip_status(err);
}

int moe_w2_forward(const moe_w2_planes* p, int T, int top_k, const void* x, const int32_t* topk_ids,
                   const float* topk_w, void* y, int out_dtype, void* workspace,
                   size_t workspace_bytes, int path, void* stream) {
  for (int stage = MOE_W2_STAGE_ROUTE; stage <= MOE_W2_STAGE_COMBINE; ++stage) {
    int st = moe_w2_forward_stage(p, stage, T, top_k, x, topk_ids, topk_w, y, out_dtype, workspace,
                                  workspace_bytes, path, stream);
    if (st != MOE_W2_OK) return st;
  }
  return MOE_W2_OK;
}

// ------------------------------------------------------------------------------------------------
// moe_w2_forward_noalloc: moe_w2_forward with its workspace in library-owned device memory, for
// callers that cannot allocate. `scratch` is a file-scope device array; each GPU the library runs
// on holds its own copy, at its own address, until the process ends. On the host the array's name
// is only a stand-in: its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and that pointer, never the name, is what host code passes to kernels.
// ------------------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MOE_W2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, null until looked up

// Address of this device's scratch array (looked up on the device's first call), or null.
void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[device]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[device] = ptr;
  }
  return g_scratch_ptr[device];
}
}  // namespace

int moe_w2_forward_noalloc(const moe_w2_planes* p, int T, int top_k, const void* x, const int32_t* topk_ids,
                           const float* topk_w, void* y, int out_dtype, int path, void* stream) {
  if (!p || T < 0 || top_k < 1) return MOE_W2_EINVAL;
  if (top_k > 32 || !pairs_ok(T, top_k)) return MOE_W2_EUNSUPPORTED;
  const size_t need = workspace_layout(p->E, p->K, p->I, T, top_k).total;
  if (need > (size_t)MOE_W2_NOALLOC_SCRATCH_BYTES) return MOE_W2_EUNSUPPORTED;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) return MOE_W2_EHIP;
  if (device != p->device) return MOE_W2_EINVAL;   // the planes live on another device
  void* ws = scratch_ptr(device);
  if (!ws) return MOE_W2_EHIP;
  return moe_w2_forward(p, T, top_k, x, topk_ids, topk_w, y, out_dtype, ws, (size_t)MOE_W2_NOALLOC_SCRATCH_BYTES,
                        path, stream);
}

int moe_w2_forward_slots(const moe_w2_planes* p, int E, const int32_t* slot_of_expert, int T, int top_k,
                         const void* x, const int32_t* topk_ids, const float* topk_w, void* y, int out_dtype,
                         void* workspace, size_t workspace_bytes, int path, void* stream) {
  if (E < 1) return MOE_W2_EINVAL;
  if (E > (1 << 30)) return MOE_W2_EUNSUPPORTED;
  if (T > 0 && !slot_of_expert) return MOE_W2_EINVAL;
  int st = forward_check(p, T, top_k, x, topk_ids, topk_w, y, out_dtype, workspace, workspace_bytes, path);
  if (st != MOE_W2_OK || T == 0) return st;
  const Workspace ws = workspace_layout(p->E, p->K, p->I, T, top_k);
  uint8_t* wsb = (uint8_t*)workspace;
  int32_t* sids = (int32_t*)(wsb + ws.slot_ids);
  hipError_t err = launch_slot_ids(T * top_k, E, p->E, topk_ids, slot_of_expert, sids, (long long*)(wsb + ws.counters),
                                   (hipStream_t)stream);
  if (err != hipSuccess) return MOE_W2_EHIP;
  // the forward proper, on the slot ids: the planes' experts are the slots
  return moe_w2_forward(p, T, top_k, x, sids, topk_w, y, out_dtype, workspace, workspace_bytes, path, stream);
}

int moe_w4_forward(const moe_w2_planes* p, int T, int top_k, const void* x, const int32_t* topk_ids,
                   const float* topk_w, void* y, int out_dtype, void* workspace, size_t workspace_bytes,
                   int path, void* stream) {
  if (!p || (p->fmt != kFmtW4 && p->fmt != kFmtNV4)) return MOE_W2_EINVAL;
  return moe_w2_forward(p, T, top_k, x, topk_ids, topk_w, y, out_dtype, workspace, workspace_bytes, path, stream);
}

int moe_w2_read_miss_counter(const void* workspace, int64_t* miss_pairs, void* stream) {
  if (!workspace) return MOE_W2_EINVAL;
  long long c = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = hipMemcpyAsync(&c, (const long long*)workspace + 2, sizeof(c), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return MOE_W2_EHIP;
  if (miss_pairs) *miss_pairs = c;
  return MOE_W2_OK;
}

int moe_w2_read_counters(const void* workspace, int64_t* invalid_pairs, int64_t* act_overflow,
                         void* stream) {
  if (!workspace) return MOE_W2_EINVAL;
  long long c[2] = {0, 0};
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = hipMemcpyAsync(c, workspace, sizeof(c), hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return MOE_W2_EHIP;
  if (invalid_pairs) *invalid_pairs = c[0];
  if (act_overflow) *act_overflow = c[1];
  return MOE_W2_OK;
}

int nvfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* e4m3, const float* scale_2,
                uint8_t* codes, uint8_t* scales, void* stream) {
  if (n < 0 || R < 0 || C < 0) return MOE_W2_EINVAL;
  if (C % 32) return MOE_W2_EUNSUPPORTED;
  const long long nb = (long long)n * R * (C / 32);
  if (nb == 0) return MOE_W2_OK;
  if (!e2m1 || !e4m3 || !scale_2 || !codes || !scales) return MOE_W2_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  int32_t* dflag = nullptr;
  if (hipMalloc(&dflag, sizeof(int32_t)) != hipSuccess) { (void)hipGetLastError(); return MOE_W2_ENOMEM; }
  int32_t flag = 0;
  hipError_t err = hipMemsetAsync(dflag, 0, sizeof(int32_t), s);
  if (err == hipSuccess) err = launch_nvfp4_to_w2(n, R, C, e2m1, e4m3, scale_2, codes, scales, dflag, s);
  if (err == hipSuccess) err = hipMemcpyAsync(&flag, dflag, 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  (void)hipFree(dflag);
  if (err != hipSuccess) return MOE_W2_EHIP;
  return flag ? MOE_W2_ENVFP4 : MOE_W2_OK;
}

// Runs a re-quantizer launch with a device flag for invalid input (synchronous).
static int requant_call(hipStream_t s, int bad_status, hipError_t (*launch)(int32_t*, const void*), const void* ctx) {
  int32_t* dflag = nullptr;
  if (hipMalloc(&dflag, sizeof(int32_t)) != hipSuccess) { (void)hipGetLastError(); return MOE_W2_ENOMEM; }
  int32_t flag = 0;
  hipError_t err = hipMemsetAsync(dflag, 0, sizeof(int32_t), s);
  if (err == hipSuccess) err = launch(dflag, ctx);
  if (err == hipSuccess) err = hipMemcpyAsync(&flag, dflag, 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  (void)hipFree(dflag);
  if (err != hipSuccess) return MOE_W2_EHIP;
  return flag ? bad_status : MOE_W2_OK;
}

int fp8_block128_to_w2(int n, int R, int C, const uint8_t* e4m3, const float* bscale, uint8_t* codes,
                       uint8_t* scales, void* stream) {
  if (n < 0 || R < 0 || C < 0) return MOE_W2_EINVAL;
  if (R % 128 || C % 128) return MOE_W2_EUNSUPPORTED;
  if ((long long)n * R * C == 0) return MOE_W2_OK;
  if (!e4m3 || !bscale || !codes || !scales) return MOE_W2_EINVAL;
  struct Ctx { int n, R, C; const uint8_t* e; const float* b; uint8_t *c, *s; hipStream_t st; } ctx{
      n, R, C, e4m3, bscale, codes, scales, (hipStream_t)stream};
  return requant_call((hipStream_t)stream, MOE_W2_ENAN, [](int32_t* f, const void* p) {
    const Ctx& c = *static_cast<const Ctx*>(p);
    return launch_fp8_block128_to_w2(c.n, c.R, c.C, c.e, c.b, c.c, c.s, f, c.st);
  }, &ctx);
}

int mxfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* ue8m0, uint8_t* codes, uint8_t* scales,
                void* stream) {
  if (n < 0 || R < 0 || C < 0) return MOE_W2_EINVAL;
  if (C % 32) return MOE_W2_EUNSUPPORTED;
  if ((long long)n * R * C == 0) return MOE_W2_OK;
  if (!e2m1 || !ue8m0 || !codes || !scales) return MOE_W2_EINVAL;
  struct Ctx { int n, R, C; const uint8_t *e, *u; uint8_t *c, *s; hipStream_t st; } ctx{
      n, R, C, e2m1, ue8m0, codes, scales, (hipStream_t)stream};
  return requant_call((hipStream_t)stream, MOE_W2_ENAN, [](int32_t* f, const void* p) {
    const Ctx& c = *static_cast<const Ctx*>(p);
    return launch_mxfp4_to_w2(c.n, c.R, c.C, c.e, c.u, c.c, c.s, f, c.st);
  }, &ctx);
}

}  // extern "C"
