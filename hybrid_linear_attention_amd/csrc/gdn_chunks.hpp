// Where a chunk lives, on the device: fixed-length batches compute it, packed
// (varlen) batches read the table built from cu_seqlens.
#pragma once
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// The chunk table is read through the constant address space: every caller
// passes a wave-uniform chunk id, so these become scalar loads.  A vector load
// here would make any wait for it (vector loads complete in order) also wait
// for a producer's in-flight global->LDS copies.
typedef const __attribute__((address_space(4))) int32_t const_i32;

// First token (row of the packed tensors) and length of chunk `cid`; a length
// <= 0 marks an unused varlen table slot.
__device__ __forceinline__ void chunk_of(const ChunkMap& cm, int cid, int& tok0, int& L) {
  if (cm.tab) {
    const_i32* t = (const_i32*)cm.tab;
    tok0 = t[2 * cid];
    L = t[2 * cid + 1];
  } else {
    const int b = cid / cm.Nc, j = cid - (cid / cm.Nc) * cm.Nc;
    tok0 = b * cm.T + kC * j;
    L = min(kC, cm.T - kC * j);
  }
}

// The chunks of sequence `seq`: ids cid0 .. cid0 + nch - 1.
__device__ __forceinline__ void seq_chunks(const ChunkMap& cm, int seq, int& cid0, int& nch) {
  if (cm.tab) {
    const_i32* so = (const_i32*)cm.seq_off;
    cid0 = so[seq];
    nch = min(so[seq + 1], cm.nc_max) - cid0;
  } else {
    cid0 = seq * cm.Nc;
    nch = cm.Nc;
  }
}

}  // namespace gdn
