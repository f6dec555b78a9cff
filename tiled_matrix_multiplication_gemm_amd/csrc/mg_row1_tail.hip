// K-tail kernels of table row 1 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(1, Fast1)
