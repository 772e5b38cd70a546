// Return-code names of libmep.so.
#include "host_common.h"

extern "C" const char* mep_status_string(int code) {
    switch (code) {
        case MEP_OK: return "MEP_OK";
        case MEP_ERR_INVALID_ARG: return "MEP_ERR_INVALID_ARG";
        case MEP_ERR_UNSUPPORTED: return "MEP_ERR_UNSUPPORTED";
        case MEP_ERR_CAPACITY: return "MEP_ERR_CAPACITY";
        case MEP_ERR_DEVICE: return "MEP_ERR_DEVICE";
        default: return "MEP_UNKNOWN_STATUS";
    }
}
