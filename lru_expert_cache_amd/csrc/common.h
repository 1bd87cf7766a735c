// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ftmoe.h"
#include "layout.h"

namespace ftmoe {

// ------------------------------------------------------------ limits
constexpr int kMaxExperts = 512;  // per layer (LDS tables in the resolve kernel)
constexpr int kMaxTopK = 16;
constexpr int kResolveThreads = 1024;
constexpr int kGroupTok = 16;    // tokens of a group's first rows kept beside its descriptor
constexpr int kMaxSlots = 65536;  // pool slots (LDS bitmap of protected slots in resolve)

// ------------------------------------------------------------ per-call device records
struct alignas(64) GroupDesc {
  uint64_t wptr;       // device address of the expert (device layout)
  int32_t row_begin;   // first row of the group in the grouped order
  int32_t row_count;   // rows (pairs) of the group
  int32_t expert;      // expert index (E for the shared expert)
  int32_t slot;        // pool slot, -1 for host-computed, -2 for the shared expert
  // run-list entries: the tokens of the group's first kGroupTok rows (low 16
  // bits), so that a decode FFN gets its activation rows from the same load
  // as the descriptor; read only when every group has at most kGroupTok rows
  uint16_t tok[kGroupTok];
};
static_assert(sizeof(GroupDesc) == 64, "one 64-byte load per descriptor");

// Header the resolve kernel writes into mapped pinned memory for the host.
struct ResolveHeader {
  int32_t t1;            // end (exclusive) of the wave that starts at t0
  int32_t n_groups;      // distinct experts of the wave (D)
  int32_t n_hit_list;    // groups runnable at once (hits, plus the shared expert)
  int32_t n_stream;      // streamed-miss groups
  int32_t n_cpu;         // host-computed groups
  int32_t pairs;         // pairs of the wave
  int32_t rows;          // rows incl. shared-expert rows
  int32_t max_rows;      // largest group
  int32_t cpu_rows;      // rows of host-computed groups
  int32_t rows_hit_list; // rows of the groups in the hit list (incl. shared)
  int32_t rows_stream;   // rows of the streamed-miss groups
  int32_t pad;
  double min_gap;        // smallest top-k gap over the wave's tokens
  uint32_t seq;          // written last: the stamp of the wave (the host waits for it)
  uint32_t pad2;
  // followed by: int32 stream_expert[n], int32 stream_slot[n], int32 cpu_expert[n],
  // int32 cpu_row_begin[n], int32 cpu_row_count[n], int32 cpu_row_tok[rows], float cpu_row_w[rows]
};

// Counters per layer in device memory.
enum { ST_PAIR_HITS, ST_PAIR_MISSES, ST_EXPERT_HITS, ST_EXPERT_MISSES, ST_CPU_MISSES, ST_EVICTIONS,
       ST_BYTES_H2D, ST_CALLS, ST_COUNT };

// ------------------------------------------------------------ device table
struct DevTable {
  int32_t* key2slot;   // [L*E], -1 if not resident
  int32_t* slot_key;   // [C], -1 if free
  uint64_t* slot_last; // [C]
  int32_t* lru[2];     // [C] each; lru[*lru_cur] = slots: free ascending, then resident by last use
  int32_t* lru_cur;    // [1] which of the two recency buffers is current
  uint64_t* clock;     // [1]
  uint64_t* stats;     // [L][ST_COUNT]
  double* min_gap;     // [L]
};

// Arguments of the resolve / permute kernel.
struct ResolveArgs {
  const double* z;         // [T][E] router logits (read when do_topk)
  int32_t do_topk;         // 1: compute sel / w / gap of all T tokens first
  int32_t* sel;            // [T*k]
  float* w;                // [T*k]
  double* gap;             // [T]
  int32_t t0, T, k, E, layer, C, mode;  // mode 0 decode, 1 staged
  int32_t stamp;
  double share;
  int64_t expert_bytes;    // streamed bytes of one expert of this layer
  int32_t hidden;
  uint64_t arena;          // device address of slot 0
  int64_t slot_bytes;
  uint64_t shared_ptr;     // device address of the shared expert, 0 if none
  DevTable tab;
  // outputs (device)
  uint8_t* pair_flag;      // [T*k] FT_PAIR_*
  int32_t* pair_slot;      // [T*k]
  int32_t* pair_row;       // [T*k] row of pair (wave-relative)
  int32_t* row_tok;        // [rows] token of row
  float* row_w;            // [rows]
  GroupDesc* groups;       // [max groups + 1]
  int32_t* glist;          // [max groups + 1]: hit list, then streamed, then host
  GroupDesc* gdesc;        // [max groups + 1]: the descriptors in glist order
  int32_t* dev_header;     // device copy of the header counts (for early-exit kernels)
  int32_t* tiles;          // prefill: (group, 128-row tile) pairs for the MX GEMM, or null
  int32_t* row_slot;       // prefill (with tiles): each row's slot in the MX GEMM activation tiles
  int32_t tile_rows;       // rows per tile
  // mapped pinned memory for the host (decode only), may be 0
  uint8_t* host_rb;
  int64_t host_rb_cap;
  // stage-timing counters for calls whose group and row counts the host never
  // reads (device-driven decode): per timed stage (0 gate/up, 1 down, 2 copy)
  // and weight format, {expert groups, rows} are added.  Null = off.
  uint64_t* prof_cnt;      // [3][4][2]
  int32_t prof_stages;     // bit i: stage i above is timed in this call
  int32_t fmt;             // weight format of the layer
  int32_t host_wait;       // 1: the host spins on the readback stamp (publish it system-wide)
  int32_t stage_hits;      // staged calls: 1 = experts resident in the pool run from their slots
  // staged calls, spread over workgroups: per-chunk histograms and the
  // per-expert results of the resolve, see launch_resolve (null = one workgroup)
  int32_t* agg;
  int32_t nchunks;         // chunks of kStageChunk pairs
};
constexpr int kStageChunk = 1024;  // pairs per workgroup of the staged histogram / rows kernels
// ints of the staged-resolve scratch for `pairs` pairs of E experts
inline int64_t stage_agg_ints(int64_t pairs, int E) {
  return 4 * ((pairs + kStageChunk - 1) / kStageChunk) * int64_t(E) + 5 * int64_t(E);
}

// ------------------------------------------------------------ launchers
// Every launcher takes an optional pair of events (ev0, ev1).  When given, the
// kernel is launched with hipExtLaunchKernelGGL so that the events bracket the
// kernel's own execution (not the gap while the host enqueues it); either may
// be null (a stage of several kernels: the first records ev0, the last ev1).
struct Ev {
  hipEvent_t a = nullptr, b = nullptr;
};

template <typename K, typename... Args>
inline void ft_launch(K kernel, dim3 grid, dim3 block, hipStream_t s, Ev ev, Args... args) {
  if (ev.a || ev.b)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.a, ev.b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}
// the same with dynamic LDS bytes
template <typename K, typename... Args>
inline void ft_launch_lds(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Ev ev, Args... args) {
  if (ev.a || ev.b)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.a, ev.b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// router.hip
hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* bias, double* z,
                                int T, int H, int E, hipStream_t s, Ev ev = {});
hipError_t launch_topk(const double* z, int T, int E, int k, int32_t* sel, float* w, double* gap,
                       hipStream_t s, Ev ev = {});
// resolve.hip
hipError_t launch_resolve(const ResolveArgs& a, hipStream_t s, Ev ev = {});
hipError_t launch_stage_table(DevTable tab, int E, int C, int layer, int num_layers, int pairs,
                              int64_t expert_bytes, hipStream_t s);
hipError_t launch_uncommit(DevTable tab, const int32_t* keys, const int32_t* slots, int n, int C,
                           hipStream_t s);
// ffn.hip
struct FfnArgs {
  const GroupDesc* gdesc; // the groups to run, in run order (one load per group)
  int32_t n_list;         // groups to run: the smaller of this (also the grid's bound) and
  const int32_t* n_list_dev;    // the count read on the device (a constant INT32_MAX when
                                // the host knows the count)
  const uint16_t* x;      // gate/up: activations [T][H] indexed by token; down: hbuf [rows][I]
  const int32_t* row_tok; // gate/up: token of each row
  const float* row_w;     // down: routing weight of each row
  uint16_t* out;          // gate/up: hbuf [rows][I]; down: pbuf [rows][H]
  int32_t hidden, inter;
  ExpertLayout lay;
  int32_t act_mode;       // FT_ACT_* >> 4
  int32_t max_rows;       // bound on the rows of any group (a decode call's token count):
                          // <= 16 ring (gate/up), <= 64 streaming kernel; 0 = unknown
};
hipError_t launch_ffn_gateup(const FfnArgs& a, hipStream_t s, Ev ev = {});
hipError_t launch_ffn_down(const FfnArgs& a, hipStream_t s, Ev ev = {});
hipError_t launch_combine(const uint16_t* pbuf, const int32_t* pair_row, int t0, int T, int k, int H,
                          int shared_row0, uint16_t* out, hipStream_t s, Ev ev = {});
bool ffn_shape_ok(int fmt, int hidden, int inter);
const char* ffn_last_kernel(bool gateup);  // kernel of the latest gate/up or down launch

// copy.hip: streamed misses copied by the GPU from the pinned host store.
// The list is the one the resolve kernel left in device memory: entries
// glist[hdr[2] .. hdr[2] + hdr[3]) are the streamed-miss groups, whose
// GroupDesc holds the destination slot address and the expert.
struct MissCopyArgs {
  const uint8_t* host;        // device-visible address of the pinned host store
  const int64_t* key_off;     // [L*E] offset of each key's blob in the store
  const int32_t* dev_header;  // resolve's counts
  const GroupDesc* gdesc;     // groups in run order: the streamed misses from dev_header[2]
  int32_t layer, E;
  int64_t bytes;              // bytes per expert of this layer (multiple of 16)
  // copy time on the device's constant-rate wall clock: clk[0] (earliest
  // workgroup start, reset to ~0), clk[1] (latest end), clk[2] (workgroups
  // done); the last workgroup adds clk[1] - clk[0] to *ticks and resets clk.
  // Null = not measured.
  uint64_t* clk;
  uint64_t* ticks;
};
hipError_t launch_miss_copy(const MissCopyArgs& a, int workgroups, hipStream_t s, Ev ev = {});
// debug: fill the slots of the streamed misses with 0xFF bytes (FT_MOE_POISON)
hipError_t launch_poison_slots(const MissCopyArgs& a, int workgroups, hipStream_t s);
// debug (FT_MOE_DEBUG_CHECKSUM): checksum of an expert in the device layout
// (host side, the store), and a kernel that recomputes it for the groups
// g0 .. min(g1, *n_dev) - 1 of a run list before their FFN reads them and
// records the first mismatch in bad[0] = 1 + key, bad[1] = slot
uint64_t slot_checksum(const uint8_t* blob, int64_t bytes);
hipError_t launch_verify_slots(const GroupDesc* gdesc, int g0, int g1, const int32_t* n_dev, const uint64_t* key_sum,
                               int key0, int64_t bytes, uint64_t* bad, hipStream_t s);

// mxq.hip: bf16 rows [rows][K] -> MX codes (FP4 [rows][K/2] or FP8 [rows][K]) + E8M0 scales [rows][K/32]
// Activation tiles of the MX GEMM: for each (row tile, 128-K step) of the
// work list, the tile's 128 rows of quantised codes in the GEMM's B-operand
// lane order, one contiguous block per 16-row sub-tile, and their scales.
//   FP4: block (tile, kb) = 8 sub-tiles x 1 KB; lane 16q + n of sub-tile s
//        holds row 16s + n, K 128kb + 32q .. + 31 (even element in the low nibble).
//   FP8: block (tile, kb) = 8 sub-tiles x 2 KB; half h (1 KB each), lane
//        16q + n: row 16s + n, K 128kb + 64h + 16q .. + 15.
//   scales: block (tile, kb) = 128 rows x 4 bytes (the rows' scales of the
//        step's four 32-blocks), 512 bytes.
// A row's slot is tile * 128 + (row in tile) (resolve writes it per row).
// Slots past a group's end hold zeros (tile gather) or stale codes (the
// gate/up GEMM's h output covers only real rows): either way they only reach
// output rows that the GEMM does not store.
constexpr int kMxTileRows = 128;
constexpr int64_t mx_tile_code_bytes(bool fp4) { return fp4 ? 8192 : 16384; }  // per (tile, K step)
constexpr int64_t kMxTileScaleBytes = 512;                                     // per (tile, K step)
// mxq.hip: MX quantisation of bf16 rows, row-major (codes [rows][K/2] for
// FP4, [rows][K] for FP8, even element in the low nibble; scales
// [rows][K/32]); the tile gather then lays them out as activation tiles.
struct MxQuantArgs {
  const uint16_t* in;         // [rows][K] bf16
  int32_t rows, K;
  uint8_t* out_codes;
  uint8_t* out_scales;
};
hipError_t launch_mx_quant(const MxQuantArgs& a, bool fp4, hipStream_t s);
// Copies row-major quantised rows into the activation tiles: grouped row r of
// a work-list tile reads source row row_map[r] (the gate/up input x by token).
struct MxTileArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int32_t K;
  const int32_t* row_map;     // grouped row -> source row, or null: the row itself
  const GroupDesc* groups;
  const int32_t* tiles;       // (group, tile) pairs
  const int32_t* n_tiles_dev;
  int32_t max_tiles;
  uint8_t* out_codes;
  uint8_t* out_scales;
};
hipError_t launch_mx_tile_gather(const MxTileArgs& a, bool fp4, hipStream_t s);
// gemm_mx.hip: grouped prefill GEMM on the block-scaled MFMA (MXFP4 weights, MX activations)
struct MxGemmArgs {
  const GroupDesc* groups;
  const int32_t* tiles;       // (group, tile) pairs
  const int32_t* n_tiles_dev; // number of valid pairs
  int32_t max_tiles;          // grid bound
  const uint8_t* act_codes;   // MX activations: the activation tiles (the layout above)
  const uint8_t* act_scales;
  const uint16_t* act_rows;   // bf16 activations: gate/up x [T][H] (by token), down h [rows][I]
  const int32_t* row_tok;     // bf16 gate/up: token of each row; null for down
  const float* row_w;         // down: routing weight of each row
  uint16_t* out;              // gate/up: h [rows][I]; down: p [rows][H]
  // MX gate/up: when set, h is written quantised, straight into the down
  // GEMM's activation tiles (row i of the grouped order at tile slot
  // row_slot[i]; these tiles must not alias act_codes), and out is not written
  uint8_t* h_codes;
  uint8_t* h_scales;
  const int32_t* row_slot;
  int32_t hidden, inter;
  ExpertLayout lay;
};
int mx_gemm_rows_per_tile();
// act: FT_ACT_* >> 4 (0 bf16, 1 MXFP8, 2 MXFP4); weights MXFP4
hipError_t launch_mx_gemm(const MxGemmArgs& a, bool gateup, int act, hipStream_t s, Ev ev = {});

// mfma_peak.hip: register-only MFMA loops (kind 0: scaled 32x32x64 FP4, 1:
// scaled 16x16x128 FP8, 2: 16x16x32 bf16, 3: 32x32x16 bf16); out holds
// mfma_peak_out_bytes()
double mfma_peak_flops(int kind, int iters);
hipError_t launch_mfma_peak(int kind, int iters, int seed, float* out, hipStream_t s);
size_t mfma_peak_out_bytes();

// noalloc.hip: the static scratch array of ft_moe_layer_forward_noalloc (one
// per GPU).  scratch_register_device looks up its device address on `device`
// (which must be current) once; scratch_device_ptr returns the kept address
// (null before registration or after a failed one).
constexpr int64_t kScratchBytes = int64_t(16) << 20;
int scratch_register_device(int device);
uint8_t* scratch_device_ptr(int device);

// ------------------------------------------------------------ errors
void set_error(const char* fmt, ...);
const char* get_error();

}  // namespace ftmoe

#define FT_HIP_CHECK(call)                                                              \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      ::ftmoe::set_error("%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, \
                         __LINE__);                                                    \
      return FT_E_HIP;                                                                 \
    }                                                                                  \
  } while (0)
