// Host-side internals of libmoew2: the planes object, the workspace layout and the kernel
// launchers implemented in the .hip files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_w2.h"

struct moe_w2_planes {
  int E, K, I;
  int fmt;             // weight format: kFmtW2 (2-bit codes) or kFmtW4 (e2m1 codes), both UE8M0 / 32;
                       // kFmtNV4 (e2m1 codes, E4M3FN / 16, fp32 scale_2 per tensor)
  int device;
  void* base;          // single device allocation
  size_t bytes;
  uint8_t* gu_codes;   // [E][2I/16][K/256][tile code bytes: 1024 (w2) or 2048 (w4)]
  uint8_t* gu_scales;  // [E][2I/16][K/256][128]
  uint8_t* dn_codes;   // [E][K/16][I/256][tile code bytes]
  uint8_t* dn_scales;  // [E][K/16][I/256][128]   (NVFP4: 256-byte scale tiles)
  float* scale2;       // NVFP4: [E][3] fp32 scale_2 of the gate rows, the up rows and the down matrix
  int32_t* flag;       // pack-time validation flags (device)
};

namespace moew2 {

// Weight formats of the planes. W2: 2-bit sign-symmetric codes; W4: e2m1 (fp4) codes (MXFP4);
// NV4: e2m1 codes with E4M3FN scales per 16 and an fp32 scale_2 per tensor (NVFP4).
enum { kFmtW2 = 0, kFmtW4 = 1, kFmtNV4 = 2 };
inline int code_bits(int fmt) { return fmt == kFmtW2 ? 2 : 4; }
inline int scale_group(int fmt) { return fmt == kFmtNV4 ? 16 : 32; }   // values per scale byte

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Pack-time validation flags
enum { kFlagScale = 1,      // pack: a UE8M0 scale byte above 252
       kFlagNaN = 2 };     // pack (NVFP4): a NaN e4m3 scale byte or a non-finite scale_2

// Workspace layout of one forward.
struct Workspace {
  // counters: [0] invalid pairs, [1] act overflow, [2] slot misses (int64)
  size_t counters;
  size_t offsets;     // int32 [E+1]
  size_t perm;        // int32 [P]
  size_t active;      // int32 [E]   expert of each active slot
  size_t meta;        // int32 [8]   [0] = number of active experts, [1] = number of GEMM M-tiles
  size_t tiles;       // int32 [max(max_tiles, max_chunks)][2] (expert, first sorted row): the GEMM
                      // M-tiles, or the sorted decode organisation's chunks
  size_t chunk_cnt;   // int32 [nchunks][E+1] per-chunk counts (large routing)
  size_t rank;        // int32 [P] rank of a pair within its chunk and expert
  size_t xq;          // x split for the block-scaled instruction (GEMM path): one 608-byte
                      // three-part e2m3 record per (token, k-tile), layout at kA6Bytes
  size_t act;         // fp16 [P][I] gated intermediate in pair order (decode path)
  size_t aq;          // gated intermediate split (GEMM path, written by the gate_up epilogue):
                      // one 608-byte three-part e2m3 record per (sorted row, k-tile)
  size_t pair_out;    // fp32 [P][K] per-pair down outputs, indexed by pair id
  size_t gu_part;     // fp32 [kWideSlices][P][2I] gate (first I) and up partial sums of the sorted
                      // decode organisation's reduction slices, by pair id (P <= kWideMaxPairs);
                      // once they are summed, fp32 [P][K]: the second reduction half of the down
                      // stage's split groups, by pair id
  size_t pair_ncs;    // int32 [P] reduction slices of each valid pair's group (sorted organisation)
  size_t slot_ids;    // int32 [P] the ids mapped to slots (slot forward)
  size_t total;
  int P, nchunks, max_tiles, max_chunks;
};

constexpr int kRouteChunk = 256;       // pairs per routing chunk
constexpr int kRouteSmallMax = 1024;   // single-workgroup routing up to this many pairs
constexpr int kGemmBM = 64;            // GEMM M-tile (sorted pair rows)
constexpr int kDecodeChunk = 4;        // decode kernels: token rows per weight pass
constexpr int kSortedMinPairs = 384;   // AUTO path: the sorted decode organisation from this many pairs
constexpr int kDecodeMaxPairs = 512;   // AUTO path: decode kernels up to this many pairs
constexpr int kDirectMaxPairs = 8;     // decode without a routing pass up to this many pairs
constexpr int kWideSlices = 4;         // sorted decode: a group of up to 4 chunks (16 rows) of one
                                       // expert splits its gate_up reduction over this many workgroups
constexpr int kWideMaxPairs = kDecodeMaxPairs;   // ... for forwards of at most this many pairs

Workspace workspace_layout(int E, int K, int I, int T, int top_k);
size_t route_scratch_bytes(int E, int P);

// Launchers (return hipError_t of the launch)
hipError_t launch_pack_nv4(const moe_w2_planes* p, const uint8_t* gu_codes, const uint8_t* gu_scales,
                           const float* gu_scale2, const uint8_t* dn_codes, const uint8_t* dn_scales,
                           const float* dn_scale2, int unpack, hipStream_t s);
hipError_t launch_pack(const moe_w2_planes* p, const uint8_t* gu_codes, const uint8_t* gu_scales,
                       const uint8_t* dn_codes, const uint8_t* dn_scales, hipStream_t s);
hipError_t launch_pack_experts(const moe_w2_planes* p, int e0, int n, const uint8_t* gu_codes,
                               const uint8_t* gu_scales, const uint8_t* dn_codes, const uint8_t* dn_scales,
                               hipStream_t s);
// Slot forward: slot_ids[p] = slot_of_expert[ids[p]] (-1 for ids outside [0, E) and for experts
// in no slot); counters[2] = number of misses.
hipError_t launch_slot_ids(int P, int E, int S, const int32_t* ids, const int32_t* slot_of_expert,
                           int32_t* slot_ids, long long* counters, hipStream_t s);
hipError_t launch_unpack(const moe_w2_planes* p, uint8_t* gu_codes, uint8_t* gu_scales,
                         uint8_t* dn_codes, uint8_t* dn_scales, hipStream_t s);

// Routing: writes offsets/perm (+ active list, tiles, counters when the pointers are non-null).
struct RouteOut {
  int32_t* offsets;
  int32_t* perm;
  int32_t* active;    // may be null
  int32_t* meta;      // may be null
  int32_t* tiles;     // may be null
  long long* counters;  // may be null
  int32_t* chunk_cnt; // scratch for P > kRouteSmallMax
  int32_t* rank;      // scratch for P > kRouteSmallMax
  int max_tiles;
  int tile_rows;      // rows per tile of the tile list (kGemmBM or kDecodeChunk)
  int wide = 0;       // sorted decode organisation: groups of 4 tiles split along the reduction
};
hipError_t launch_route(int E, int T, int top_k, const int32_t* ids, const RouteOut& o, hipStream_t s);

// Decode path (small groups): gate_up + SiLU, down, combine. Organisations:
//  kDecodeRouted - each workgroup row finds its expert's pairs from the ids (no routing pass);
//  kDecodeDirect - P <= kDirectMaxPairs, one group per pair; the down launch also writes y;
//  kDecodeSorted - workgroup rows walk the chunk list of a routing pass (kDecodeChunk rows per
//                  chunk, in expert order), so one expert's chunks run together; with the wide
//                  list (P <= kWideMaxPairs) groups of 4 chunks share one weight pass (split
//                  gate_up reduction, 8-row down).
enum { kDecodeRouted = 0, kDecodeDirect = 1, kDecodeSorted = 2 };
hipError_t launch_decode_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                                 const int32_t* ids, const Workspace& ws, uint8_t* wsb, int mode,
                                 hipStream_t s);
hipError_t launch_decode_down(const moe_w2_planes* p, int T, int top_k, const int32_t* ids, const float* w,
                              void* y, int out_dtype, const Workspace& ws, uint8_t* wsb, int mode,
                              hipStream_t s);
size_t decode_direct_lds(int I);
// GEMM path (large groups)
hipError_t launch_gemm_gate_up(const moe_w2_planes* p, int T, int top_k, const void* x,
                               const Workspace& ws, uint8_t* wsb, hipStream_t s);
hipError_t launch_gemm_down(const moe_w2_planes* p, int T, int top_k, const Workspace& ws,
                            uint8_t* wsb, hipStream_t s);
// pair_ncs, pair_out2: the sorted decode organisation's wide list (split down groups), else null
hipError_t launch_combine(int T, int top_k, int E, int K, const int32_t* ids, const float* w,
                          const float* pair_out, void* y, int out_dtype, hipStream_t s,
                          const int32_t* pair_ncs = nullptr, const float* pair_out2 = nullptr);

// Re-quantizers
hipError_t launch_fp8_block128_to_w2(int n, int R, int C, const uint8_t* e4m3, const float* bscale,
                                     uint8_t* codes, uint8_t* scales, int32_t* flag, hipStream_t s);
hipError_t launch_mxfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* ue8m0, uint8_t* codes,
                              uint8_t* scales, int32_t* flag, hipStream_t s);
hipError_t launch_nvfp4_to_w2(int n, int R, int C, const uint8_t* e2m1, const uint8_t* e4m3,
                              const float* scale_2, uint8_t* codes, uint8_t* scales, int32_t* flag,
                              hipStream_t s);

}  // namespace moew2
