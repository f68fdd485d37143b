// Host-side view of the persistent kernels: the parameter block every launch
// takes and the launch entry points implemented in kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "comm_units.hpp"
#include "gemm_tile.hpp"
#include "schedule.hpp"

namespace iris {

enum OpKind : int32_t {
  OP_GEMM = 0,        // GEMM queue only (no comm units)
  OP_AG = 1,          // comm: all_gather copy units; GEMM waits on row flags
  OP_RS = 2,          // comm: reduce_scatter units wait on GEMM tile flags
  OP_ARMM = 3,        // comm: matmul_all_reduce units wait on GEMM tile flags
  OP_CONC_AR = 4,     // comm: independent flat reduce units (all_reduce, reduce_scatter)
  OP_CONC_COPY = 5,   // comm: independent block copies (all_gather, all_to_all,
                      // broadcast, matmul_all_gather's peer blocks)
};

// Workspace layout: first uint64 stamps[kMaxGrid][4] written by the
// persistent kernel, uint64 comm_stamps[kMaxGrid][2] written by the
// sequential-mode comm kernel and uint64 clocks[kMaxGrid][4] (shader-clock
// and 100 MHz counters at entry and exit of each persistent workgroup), a
// fixed-size block of kStampWords words, then the int32 words
//   GEMM queue counters (one per XCD), comm queue counter, error word (set
//   by a wait that gave up during this launch), finished-workgroup counter,
//   finished comm units (all_gather), status word, finished tiles of each
//   XCD queue (the lockstep of the GEMM rounds), then from kFlagBase the
//   ready words: all_gather, one counter per GEMM row block (finished copy
//   units of that block, kLine words apart); reduce, one flag per GEMM tile
// Every word but the status word is zero when a persistent launch starts;
// the last workgroup to finish folds the error word into the status word and
// zeroes the rest again, so consecutive ops on one workspace need no
// separate reset. The status word keeps its bits until the host reads and
// clears it (iris_check_device_error).
// Each counter sits on its own 128-byte line (kLine words), and so does each
// all_gather row-block counter: many workgroups poll these while others bump
// them, and words sharing a line would serialise both.
constexpr int kLine = 32;
constexpr int kCtrGemm = 0;  // kXcds GEMM queue counters, one line each
constexpr int kCtrComm = kXcds * kLine, kErr = kCtrComm + kLine, kDone = kErr + kLine,
              kCommDone = kDone + kLine, kStatus = kCommDone + kLine;
constexpr int kTileDone = kStatus + kLine;  // finished tiles of each XCD queue, one line each
constexpr int kFlagBase = kTileDone + kXcds * kLine;
// bits of the status word
constexpr int kStatusTimeout = 1;
constexpr int kMaxGrid = 2048;
constexpr int kClockOff = 6;    // clocks start at stamps + kMaxGrid * kClockOff
constexpr int kStampWords = 10; // uint64 words per workgroup slot in the stamp block

struct Params {
  GemmArgs g;
  CommArgs c;
  int32_t op;
  TileOrder order;           // GEMM tile grid and visiting order
  int32_t xcd_q;             // tiles per block dealt to each XCD queue
  int32_t T_gemm, T_comm;
  int32_t gemm_wgs;          // pid < gemm_wgs starts on the GEMM queue
  int32_t steal;             // switch to the other queue when the first is empty
  int32_t lockstep;          // the tiles of round r of an XCD queue start after round r-1 has finished
  int32_t fused;             // 1: flags are produced and awaited in this launch
  int32_t* ws;               // counters + flags
  uint64_t* stamps;          // [gridDim.x][4]: gemm start/end, comm start/end
  uint64_t* comm_stamps;     // [gridDim.x][2]: comm-only kernel start/end
  uint32_t spin_limit;       // bound on polls of one flag wait
  int32_t n_reset;           // words [0, n_reset) (except kStatus) to zero at the end
};

// Bytes of the static device scratch behind iris_ag_mm_noalloc.
constexpr size_t kScratchBytes = (size_t)1 << 20;
hipError_t scratch_setup(int dev, hipStream_t s, void** out);
void* scratch_if_set_up(int dev);

hipError_t launch_persistent(const Params& p, int bm, int bn, int grid, hipStream_t s);
hipError_t launch_comm_only(const Params& p, int grid, hipStream_t s);
// the persistent kernel's copy workgroups alone (op OP_AG, T_gemm = 0), under
// its own kernel name
hipError_t launch_gather_only(const Params& p, int bm, int bn, int grid, hipStream_t s);
// workgroups of the persistent kernel resident per CU, or <= 0 on error
int persistent_blocks_per_cu(int bm, int bn, int op);
bool tile_supported(int bm, int bn);

}  // namespace iris
