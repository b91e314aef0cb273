// Status strings of the C ABI.
#include "ev_internal.h"

EV_API const char *ev_status_string(ev_status s) {
  switch (s) {
    case EV_OK: return "ok";
    case EV_ERR_NULL: return "a required pointer is NULL";
    case EV_ERR_SHAPE: return "a size argument is out of range";
    case EV_ERR_DTYPE: return "unsupported element type";
    case EV_ERR_WORKSPACE: return "workspace is missing or too small";
    case EV_ERR_ARG: return "invalid scalar argument";
    case EV_ERR_LAUNCH: return "kernel launch failed";
    case EV_ERR_SCRATCH: return "the call needs more than the fixed scratch of the no-allocation entry point";
    case EV_DERR_PARENT: return "parent[] is not a topological tree rooted at node 0";
    case EV_DERR_BOUNDS: return "prefix and tree do not fit the cache, or a block id is out of range";
    case EV_DERR_TOKEN: return "a draft token id is outside [0, V)";
    case EV_DERR_PATH: return "path / accept_len is not a valid root path";
    case EV_DERR_WIDTH: return "a node has more children than max_children";
    default: return "unknown status";
  }
}
