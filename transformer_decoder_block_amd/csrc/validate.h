// Host side of libblock that needs no GPU: the checks of every entry point's
// arguments, the workspace layout and the rotary table.  Plain C++ with no
// HIP, so that it also builds with the host compiler under the address and
// undefined-behaviour sanitizers.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/libblock.h"

namespace blkv {

// Record msg as this thread's last error and return s.
blk_status fail(blk_status s, const std::string& msg);
const char* last_error();
const char* status_str(blk_status s);

size_t esize(int dtype);  // bytes per element of the model dtype
bool aligned16(const void* p);
// Row stride of the dense MLP's neuron buffer: the width rounded up to 64
// elements, so that each 128-byte K stage of the down projection's A rows is
// one cache line (the pad columns are never read).
size_t neuron_ld(int I);

blk_status check_config(const blk_config* c);
// io against a configuration: pointers set, distinct and 16-byte aligned,
// batch and seq within [1, max_batch] x [1, max_seq].
blk_status check_io(const blk_config& c, const blk_io* io);
blk_status check_weights(const blk_config& c, const blk_weights* w);
blk_status check_taps(const blk_config& c, const blk_taps* t);  // t may be NULL
blk_status check_forward(const blk_config& c, const blk_io* io, const blk_weights* w,
                         const blk_taps* t);

// Workspace parts, laid out in this order (those a configuration does not
// use are absent).
enum WsPart {
  WS_A, WS_Q, WS_K, WS_VT, WS_GATE, WS_PREMIX, WS_O, WS_MID, WS_M, WS_LAYER_OUT,
  WS_NEUR, WS_MLP_RAW, WS_LOGITS, WS_EIDX, WS_EW, WS_GCNT, WS_GOFF, WS_HIST,
  WS_ROW_TOKEN, WS_PAIR_ROW, WS_ROW_WEIGHT, WS_STAGE, WS_NSH, WS_ROPE_COS,
  WS_ROPE_SIN, WS_SPLIT, WS_NPARTS
};
constexpr size_t WS_ABSENT = ~(size_t)0;
struct WsLayout {
  size_t off[WS_NPARTS];    // byte offset of each part, WS_ABSENT if unused
  size_t bytes[WS_NPARTS];  // bytes each part needs (0 if unused)
  size_t total;             // sum of the parts, each rounded up to 256 bytes
};
// Layout for c.max_batch * c.max_seq tokens.  hist_ints: the dispatch
// histogram's size in ints (MoE only); split_bytes: the GEMMs' K-split
// scratch.  c must have passed check_config.
void ws_layout(const blk_config& c, size_t hist_ints, size_t split_bytes, WsLayout* L);

// Rotary table of S positions, S * head_dim / 2 floats each:
// phi[s, i] = s * theta^(-2i / head_dim) in double, cos and sin rounded to
// float (granite sheet, section "Implementing it": rotate-half rotary).
void rope_table(const blk_config& c, int S, float* cs, float* sn);

}  // namespace blkv
